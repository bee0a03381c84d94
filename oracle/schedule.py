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
