"""Nano-batch plan templates and plan JSON parsing (host logic; plans run in libnanoflow).

A plan lists nano-operations (kind, nano-batch, stream) in issue order. Templates:

* ``sequential(bounds)`` — one stream, nano-batches one after another (nano-batching
  without overlap; with one nano-batch this is the plain sequential layer).
* ``overlap(bounds, ...)`` — the 8B pipeline of the NanoFlow slides ("8B Pipeline Design":
  split into nano-batches, reorder, overlap decode attention of one nano-batch with the
  dense operations of another): a compute stream runs KQV of every nano-batch first, then
  O and Up/Gate/Down per nano-batch; a memory stream runs decode attention (and by default
  prefill attention) per nano-batch as soon as its KQV is done.
"""

from __future__ import annotations

import json

from . import abi
from .abi import NF_OP_DECATTN, NF_OP_KQV, NF_OP_O, NF_OP_PFATTN, NF_OP_UGD, HostPlan


def even_bounds(n_tokens: int, n_nano: int, granularity: int = 128) -> list:
    """Split [0, T) into n_nano nano-batches of near-equal size, cut at multiples of granularity."""
    if n_nano <= 1:
        return [0, n_tokens]
    cuts = []
    for j in range(1, n_nano):
        c = round(n_tokens * j / n_nano / granularity) * granularity
        cuts.append(min(max(c, 1), n_tokens - 1))
    b = [0] + sorted(set(cuts)) + [n_tokens]
    return b


def dag(batch: abi.HostBatch, bounds) -> dict:
    """{(kind, nano): set of (kind, nano) it depends on}, from the library's DAG builder.

    Parent dependencies only run from lower to higher kind index (KQV, attention, O, UGD),
    so a kind-major listing on one stream is always a valid order to ask about.
    """
    n = len(bounds) - 1
    ops = [(k, j, 0) for k in range(abi.NF_OP_KINDS) for j in range(n)]
    edges, _ = abi.nf_plan_dependencies(batch, HostPlan(bounds, ops, 1))
    deps = {(k, j): set() for k, j, _ in ops}
    for i, j in edges:
        deps[ops[j][:2]].add(ops[i][:2])
    return deps


def schedule(batch: abi.HostBatch, bounds, stream_of, rank, n_streams: int, cu_masks=None) -> HostPlan:
    """Plan whose listed order is a topological order of the DAG, taking among ready
    nano-ops the one of least ``rank(kind, nano)``; streams from ``stream_of(kind, nano)``.
    Every stream's order is then a subsequence of one topological order: no deadlock."""
    deps = dag(batch, bounds)
    done, ops = set(), []
    while len(ops) < len(deps):
        ready = [op for op in deps if op not in done and deps[op] <= done]
        pick = min(ready, key=lambda op: rank(*op))
        done.add(pick)
        ops.append((pick[0], pick[1], stream_of(*pick)))
    return HostPlan(bounds, ops, n_streams, cu_masks)


def sequential(batch: abi.HostBatch, bounds) -> HostPlan:
    """One stream; nano-batch by nano-batch, deferring an O/UGD whose rows wait on a
    prefill chunk that ends in a later nano-batch."""
    return schedule(batch, bounds, lambda k, j: 0, lambda k, j: (j, k), 1)


def overlap(batch: abi.HostBatch, bounds, compute_mask=None, memory_mask=None,
            prefill_on_memory: bool = True, unmasked_kinds=(), memory_kinds=()) -> HostPlan:
    """Two streams (0 compute, 1 memory): KQV of every nano-batch first on the compute
    stream, then O and Up/Gate/Down per nano-batch; decode attention per nano-batch on
    the memory stream (prefill attention there too unless prefill_on_memory is False).

    unmasked_kinds: dense kinds (NF_OP_KQV, NF_OP_O, NF_OP_UGD) that run on a third,
    unmasked stream beside the memory stream's mask instead of on the compute mask; the
    dense ops stay one lane (one at a time, in order) across the two compute streams.

    memory_kinds: dense kinds issued on the memory stream right after their nano-batch's
    attention instead of on the compute stream (a product that runs poorly beside decode
    attention then never runs beside it)."""
    third = bool(unmasked_kinds)
    if third and memory_kinds:
        raise ValueError("unmasked_kinds and memory_kinds do not combine")

    def stream_of(k, j):
        if k == NF_OP_DECATTN or (k == NF_OP_PFATTN and prefill_on_memory) or k in memory_kinds:
            return 1
        return 2 if k in unmasked_kinds else 0

    def rank(k, j):
        if k == NF_OP_KQV:
            return (0, j, 0)
        if k in (NF_OP_DECATTN, NF_OP_PFATTN) or k in memory_kinds:
            return (1, j, k)
        return (2, j, k)

    masks = None
    full = [0xFFFFFFFF] * abi.NF_CU_MASK_WORDS
    if compute_mask is not None or memory_mask is not None:
        masks = [compute_mask or full, memory_mask or full] + ([full] if third else [])
    plan = schedule(batch, bounds, stream_of, rank, 3 if third else 2, masks)
    if not third:
        return plan
    lanes = [1 if s == 1 else 0 for s in plan.stream.tolist()]
    return HostPlan(bounds, plan.ops, 3, masks, 0, lanes)


def from_json(text: str) -> tuple[HostPlan, dict]:
    """Parse a plan written by nf_plan_search (returns the plan and the whole record)."""
    rec = json.loads(text)
    ops = [(o["kind"], o["nano"], o["stream"]) for o in rec["ops"]]
    lanes = [o["lane"] for o in rec["ops"]] if all("lane" in o for o in rec["ops"]) else None
    masks = rec.get("cu_masks")
    return HostPlan(rec["bounds"], ops, rec["n_streams"], masks, rec.get("decode_grid", 0), lanes), rec
