"""Oracle of the nano-operation dependency rule and of pipeline schedules — TEST
INFRASTRUCTURE ONLY.

Follows the NanoFlow summary page, "Auto-Search Stage I": a nano-operation B depends on a
nano-operation A if and only if their parent operations are dependent in the model and
their token ranges intersect (the page's example: O1 on tokens 0-767 depends on Attn1 on
0-767 but not on Attn2 on 768-2048). Parent operations of the layer, in the order the page
and the slides list them: KQV generation, decode attention, prefill attention, O
projection, Up/Gate/Down.

Readings (the pages leave these to the model's graph): decode attention of a nano-batch
covers the decode tokens in it; prefill attention of a chunk belongs to the nano-batch
holding the chunk's last token and its range is the whole chunk, since it needs every
query and key of the chunk.

Written with plain Python sets of token rows, independent of the library's interval code.
Pins: the page's O1/Attn example and hand-built cases in the not-gpu tests.
"""

from __future__ import annotations

KQV, DECATTN, PFATTN, O, UGD = range(5)
KIND_NAMES = ("KQV", "DECATTN", "PFATTN", "O", "UGD")
PARENTS = {DECATTN: {KQV}, PFATTN: {KQV}, O: {DECATTN, PFATTN}, UGD: {O}}


def _requests(batch):
    """(first row, last row + 1, is_decode) of each request in dense-batch order."""
    out = []
    t = 0
    for _ in range(len(batch.decode_ctx)):
        out.append((t, t + 1, True))
        t += 1
    for q in batch.prefill_len:
        out.append((t, t + int(q), False))
        t += int(q)
    return out


def op_rows(batch, bounds, kind: int, j: int) -> set:
    lo, hi = bounds[j], bounds[j + 1]
    if kind in (KQV, O, UGD):
        return set(range(lo, hi))
    rows = set()
    for s, e, dec in _requests(batch):
        if kind == DECATTN and dec and lo <= s < hi:
            rows.add(s)
        if kind == PFATTN and not dec and lo <= e - 1 < hi:
            rows |= set(range(s, e))
    return rows


def dependencies(batch, bounds) -> set:
    """{((kind_a, nano_a), (kind_b, nano_b)) : B depends on A}."""
    n = len(bounds) - 1
    rows = {(k, j): op_rows(batch, bounds, k, j) for k in range(5) for j in range(n)}
    deps = set()
    for (kb, jb), rb in rows.items():
        for (ka, ja), ra in rows.items():
            if ka in PARENTS.get(kb, ()) and ra & rb:
                deps.add(((ka, ja), (kb, jb)))
    return deps


# --------------------------------------------------------------------------------------
# durations, list-schedule simulation, brute-force two-stage search
# --------------------------------------------------------------------------------------
#
# Follows "Auto-Search Stage I" (structure under no interference: number of nano-batches,
# sizes in multiples of the granularity summing to the dense batch, ordering; nano-ops of
# one class never overlap; each nano-op takes its profiled best time) and "Auto-Search
# Stage II" (structure fixed; an op's time is its best time divided by its normalised
# performance P under the chosen resource split). Readings (no MILP is given on the pages):
# one in-order stream per class (compute: KQV, O, UGD; memory: decode attention; prefill
# attention on either), orders drawn from a KQV-lookahead family, profiled times
# interpolated linearly in the nano-batch size, and P depending only on whether an op of
# the other class is running. A configuration gives (P_gemm_both, P_mem_both,
# P_gemm_alone, P_mem_alone).

def interp(points, x):
    """Piecewise-linear through (size, ms) points; through the origin below the first,
    extended along the last segment above the last."""
    if x <= 0 or not points:
        return 0.0
    pts = sorted(points)
    if x <= pts[0][0]:
        return pts[0][1] * x / pts[0][0]
    for (x0, y0), (x1, y1) in zip(pts, pts[1:]):
        if x <= x1:
            return y0 + (y1 - y0) * (x - x0) / (x1 - x0)
    if len(pts) == 1:
        return pts[0][1] * x / pts[0][0]
    (x0, y0), (x1, y1) = pts[-2], pts[-1]
    return y1 + (y1 - y0) * (x - x1) / (x1 - x0)


def durations(batch, bounds, table):
    """Best time of every nano-op (kind, nano) from a D_best table {kind: [(size, ms)]}."""
    n = len(bounds) - 1
    reqs = _requests(batch)
    out = {}
    for j in range(n):
        lo, hi = bounds[j], bounds[j + 1]
        out[(KQV, j)] = interp(table["KQV"], hi - lo)
        out[(O, j)] = interp(table["O"], hi - lo)
        out[(UGD, j)] = interp(table["UGD"], hi - lo)
        n_dec = sum(1 for s, e, dec in reqs if dec and lo <= s < hi)
        out[(DECATTN, j)] = interp(table.get("DECATTN", []), n_dec)
        out[(PFATTN, j)] = sum(interp(table.get("PFATTN", []), e - s) for s, e, dec in reqs
                               if not dec and lo <= e - 1 < hi)
    return out


def simulate(streams, deps, dur, speeds=None, full=None, full_kinds=()):
    """Makespan of in-order streams (lists of (kind, nano)) with dependency waits.

    speeds: None (every op at full speed) or a dict with p_gemm_both, p_mem_both,
    p_gemm_alone, p_mem_alone, and optionally p_gemm_both_kind / p_gemm_alone_kind /
    p_mem_both_kind: the compute speeds of the KQV, O and UGD ops, and the memory op's speed
    beside each of them, measured one compute kind at a time against the memory op (the
    pages' pairwise interference profile, taken per compute kind; a kind without an entry
    uses the plain speed). Stream 0 is the compute stream. Returns None on
    deadlock. Time advances from one completion to the next; a running op progresses at its
    speed.

    full, full_kinds: a second speed dict and the compute kinds that take it (the pages'
    per-operation resource share: those kinds run with their own share, here the whole
    GPU beside the memory op's mask); while such a kind runs, the memory op's speed beside
    it comes from `full` too. The memory op alone keeps `speeds`.
    """
    pos = [0] * len(streams)
    cur = [None] * len(streams)
    left = [0.0] * len(streams)
    end = {}
    t = 0.0
    total = sum(len(s) for s in streams)
    while len(end) < total:
        progress = True
        while progress:  # zero-length ops may unblock another stream's head: repeat
            progress = False
            for s, ops in enumerate(streams):
                while cur[s] is None and pos[s] < len(ops):
                    op = ops[pos[s]]
                    if not all(d in end and end[d] <= t for d in deps.get(op, ())):
                        break
                    pos[s] += 1
                    progress = True
                    if dur[op] <= 0:
                        end[op] = t
                        continue
                    cur[s], left[s] = op, dur[op]
        running = [s for s in range(len(streams)) if cur[s] is not None]
        if not running:
            if len(end) == total:
                break
            return None  # deadlock: a stream head waits on an op that can never run
        rate = {}
        for s in running:
            if speeds is None or len(streams) == 1:
                rate[s] = 1.0
            else:
                both = len(running) > 1
                key = ("p_gemm_" if s == 0 else "p_mem_") + ("both" if both else "alone")
                # the compute op's own placement decides its speeds, and the memory op's
                # beside it; the memory op alone runs at the plain entry's speed
                sp = speeds
                if full is not None and cur[0] is not None and cur[0][0] in full_kinds and (s == 0 or both):
                    sp = full
                rate[s] = sp[key]
                per_kind = sp.get(key + "_kind") or {}
                # the compute stream's own kind; the memory stream's speed beside it is keyed
                # by the kind of the compute op running next to it
                name = KIND_NAMES[cur[s][0]] if s == 0 else (KIND_NAMES[cur[0][0]] if both else None)
                if name in per_kind:
                    rate[s] = per_kind[name]
        dt = min(left[s] / rate[s] for s in running)
        t += dt
        for s in running:
            left[s] -= dt * rate[s]
            if left[s] <= 1e-12 * max(1.0, dur[cur[s]]):
                end[cur[s]] = t
                cur[s] = None
    return max(end.values()) if end else 0.0


def structure(n, lookahead, pf_on_memory):
    """Per-stream orders: compute = KQV_0..KQV_{a-1}, then per nano-batch j: (prefill
    attention,) O_j, UGD_j, KQV_{j+a}; memory = decode attention (and prefill) per j."""
    comp = [(KQV, j) for j in range(min(lookahead, n))]
    mem = []
    for j in range(n):
        if not pf_on_memory:
            comp.append((PFATTN, j))
        comp += [(O, j), (UGD, j)]
        if j + lookahead < n:
            comp.append((KQV, j + lookahead))
        mem.append((DECATTN, j))
        if pf_on_memory:
            mem.append((PFATTN, j))
    return [comp, mem]


def all_bounds(T, n, gran):
    """Every split of [0, T) into n nano-batches cut at multiples of gran."""
    import itertools

    cuts = list(range(gran, T, gran))
    for c in itertools.combinations(cuts, n - 1):
        yield [0, *c, T]


def _partner(c, configs):
    """The entry measured with the compute op unmasked beside the same memory mask as the
    masked entry c (same r_mem, "gemm_full" true), or None."""
    if c is None or c.get("gemm_full") or c.get("cu_masks") is None:
        return None
    for f in configs:
        if f.get("gemm_full") and f.get("cu_masks") is not None and abs(f.get("r_mem", -1) - c.get("r_mem", -1)) < 1e-6:
            return f
    return None


def placements(c, configs):
    """Stage II's per-kind choices for entry c: (full entry, kinds placed unmasked). Every
    compute kind on the complement mask, and with a partner entry each mixed subset of
    {KQV, O, UGD} (all three unmasked is the partner entry itself, searched on its own)."""
    out = [(None, ())]
    f = _partner(c, configs)
    if f is not None:
        import itertools

        for n in (1, 2):
            for kinds in itertools.combinations((KQV, O, UGD), n):
                out.append((f, kinds))
    return out


def search(batch, table, configs=None, max_nano=4, gran=128, top_k=8, min_gain=0.0):
    """Brute force over the same space as the library: Stage I by exhaustive enumeration,
    Stage II over the interference configurations (and, per masked configuration, every
    placement of the compute kinds on its complement mask or the whole GPU) for the K best
    structures and the sequential single-stream plan; an overlapped plan wins only when it
    beats the sequential one by more than the fraction min_gain. Returns (best makespan,
    stage-I best makespan)."""
    T = sum(e - s for s, e, _ in _requests(batch))
    cands = []
    for n in range(1, max_nano + 1):
        for bounds in all_bounds(T, n, gran):
            deps = {}
            for a, b in dependencies(batch, bounds):
                deps.setdefault(b, set()).add(a)
            dur = durations(batch, bounds, table)
            for look in range(1, n + 1):
                for pfm in (False, True):
                    st = structure(n, look, pfm)
                    ms = simulate(st, deps, dur)
                    if ms is not None:
                        cands.append((ms, n, bounds, st, deps, dur))
    cands.sort(key=lambda c: (c[0], c[1]))
    stage1 = cands[0][0]
    seq_bounds = [0, T]
    seq_deps = {}
    for a, b in dependencies(batch, seq_bounds):
        seq_deps.setdefault(b, set()).add(a)
    seq_dur = durations(batch, seq_bounds, table)
    seq = simulate([[(k, 0) for k in range(5)]], seq_deps, seq_dur)
    best = seq
    for ms, n, bounds, st, deps, dur in cands[:top_k]:
        for c in (configs or [None]):
            for f, kinds in placements(c, configs or []):
                r = simulate(st, deps, dur, c, f, kinds)
                if r is not None and r < best:
                    best = r
    if best > seq * (1.0 - min_gain):
        best = seq
    return best, stage1
