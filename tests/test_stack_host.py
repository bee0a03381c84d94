"""Host-side checks of the layer-stack DAG (no GPU).

A stack call runs n_layers layers over one batch on shared row buffers (h, qkv, attention
output, x1, h2, a), per-GEMM split-K workspaces, per-nano-batch split-KV partials, one KV
pool per layer and the in-place output y. These tests model every nano-op's reads and
writes of those buffers (by token rows) and check that any two ops that conflict — same
buffer, overlapping rows, at least one write — are ordered by a dependency path, that the
issue order is topological and keeps each stream's listing, and that pipelining moves the
next layer's KQV up to just after the producing Up/Gate/Down.
"""

import itertools

import numpy as np
import pytest

from synth import workloads as sw

KINDS = ("KQV", "DEC", "PF", "O", "UGD")


@pytest.fixture(scope="module")
def abi():
    from nano_intra_overlap_amd import abi as a

    a.load()
    return a


def _rows(b, bounds, kind, j):
    """Token rows an op of kind `kind` in nano-batch j covers."""
    lo, hi = bounds[j], bounds[j + 1]
    n_dec = b.n_decode
    if kind in (0, 3, 4):
        return set(range(lo, hi))
    if kind == 1:
        return set(range(min(lo, n_dec), min(hi, n_dec)))
    rows = set()
    t = n_dec
    for L in b.prefill_len:
        t0, t1 = t, t + int(L)
        if lo <= t1 - 1 < hi:  # a prefill chunk belongs to the nano-batch of its last token
            rows |= set(range(t0, t1))
        t = t1
    return rows


def _accesses(b, bounds, op_index, kind, j, layer, alias_x):
    """(buffer, rows, is_write) of one nano-op; rows None = the whole buffer."""
    R = _rows(b, bounds, kind, j)
    x = "y" if (layer > 0 or alias_x) else "x_in"
    pool = f"pool{layer}"
    ws = f"ws{op_index}"  # split-K workspace region of this op (shared by every layer)
    if kind == 0:
        return [(x, R, 0), ("h", R, 1), ("h", R, 0), ("qkv", R, 1), (pool, R, 1), (ws, None, 1)]
    if kind == 1:  # an op without rows launches nothing; it also appends its decode tokens' K/V
        return [("qkv", R, 0), (pool, R, 0), ("attn", R, 1), (f"part{j}", None, 1), (f"part{j}", None, 0),
                (pool, R, 1)] if R else []
    if kind == 2:
        return [("qkv", R, 0), (pool, R, 0), ("attn", R, 1)] if R else []
    if kind == 3:
        return [("attn", R, 0), (x, R, 0), ("x1", R, 1), (ws, None, 1)]
    return [("x1", R, 0), ("h2", R, 1), ("a", R, 1), ("y", R, 1), (ws, None, 1)]


def _check_stack(abi, b, plan, bounds, n_layers, flags, alias_x):
    hb = abi.HostBatch.from_batch(b)
    edges, listing, order = abi.nf_stack_dependencies(hb, plan, n_layers, flags)
    ops = plan.ops if plan is not None else [(k, 0, 0) for k in range(abi.NF_OP_KINDS)]
    n = len(ops)
    N = n * n_layers
    assert sorted(listing) == list(range(N)) and sorted(order) == list(range(N))
    # reachability
    reach = np.zeros((N, N), bool)
    for i, j in edges:
        reach[i, j] = True
    for k in range(N):
        reach |= reach[:, [k]] & reach[[k], :]
    pos = {op: p for p, op in enumerate(order)}
    for i, j in edges:
        assert pos[i] < pos[j], "issue order is not topological"
    # each stream takes its ops in listing order
    for s in range(max(o[2] for o in ops) + 1):
        in_listing = [op for op in listing if ops[op % n][2] == s]
        in_order = [op for op in order if ops[op % n][2] == s]
        assert in_listing == in_order
    # every conflicting pair is ordered, in the sequential program's direction
    seq = sorted(range(N), key=lambda op: (op // n, ops[op % n][0], ops[op % n][1]))
    acc = {op: _accesses(b, bounds, op % n, ops[op % n][0], ops[op % n][1], op // n, alias_x) for op in range(N)}
    for ia, a in enumerate(seq):
        for c in seq[ia + 1:]:
            conflict = any(
                ba == bc and (wa or wc) and (ra is None or rc is None or (ra & rc))
                for (ba, ra, wa), (bc, rc, wc) in itertools.product(acc[a], acc[c]))
            if conflict:
                assert reach[a, c], (f"layer {a // n} {KINDS[ops[a % n][0]]}{ops[a % n][1]} and layer {c // n} "
                                     f"{KINDS[ops[c % n][0]]}{ops[c % n][1]} conflict but are not ordered")
    return edges, listing, order, ops


def _cases(abi):
    from nano_intra_overlap_amd import plans

    rng = np.random.default_rng(5)
    for trial in range(10):
        dec = rng.integers(0, 60, int(rng.integers(1, 30)))
        pre = rng.integers(1, 50, int(rng.integers(0, 3)))
        b = sw.batch_from_lengths(dec, pre, None, seed=trial)
        hb = abi.HostBatch.from_batch(b)
        T = b.n_tokens
        n = int(rng.integers(1, min(4, T) + 1))
        bounds = [0] + sorted(rng.choice(np.arange(1, T), size=n - 1, replace=False).tolist()) + [T]
        yield trial, b, None, [0, T]
        yield trial, b, plans.sequential(hb, bounds), bounds
        yield trial, b, plans.overlap(hb, bounds), bounds
        yield trial, b, plans.overlap(hb, bounds, prefill_on_memory=False), bounds


@pytest.mark.parametrize("flags", [0, 1])
def test_stack_conflicts_are_ordered(abi, flags):
    for trial, b, plan, bounds in _cases(abi):
        for alias_x in (False, True):
            _check_stack(abi, b, plan, bounds, 3, flags, alias_x)


def test_one_layer_stack_is_the_layer(abi):
    for trial, b, plan, bounds in _cases(abi):
        hb = abi.HostBatch.from_batch(b)
        e1, o1 = abi.nf_plan_dependencies(hb, plan)
        es, ls, os_ = abi.nf_stack_dependencies(hb, plan, 1, 0)
        assert sorted(e1) == sorted(es) and o1 == os_ and ls == list(range(len(ls)))


def test_pipelining_moves_next_kqv_up(abi):
    from nano_intra_overlap_amd import plans

    b = sw.batch_from_lengths(np.full(200, 40), [56], seed=0)
    hb = abi.HostBatch.from_batch(b)
    bounds = [0, 128, b.n_tokens]
    plan = plans.overlap(hb, bounds)
    n = len(plan.ops)
    idx = {op[:2]: i for i, op in enumerate(plan.ops)}
    K0, K1 = idx[(abi.NF_OP_KQV, 0)], idx[(abi.NF_OP_KQV, 1)]
    O1, U0, U1 = idx[(abi.NF_OP_O, 1)], idx[(abi.NF_OP_UGD, 0)], idx[(abi.NF_OP_UGD, 1)]
    _, flat, _ = abi.nf_stack_dependencies(hb, plan, 3, 0)
    _, piped, order = abi.nf_stack_dependencies(hb, plan, 3, abi.NF_STACK_PIPELINE)
    at = {op: p for p, op in enumerate(piped)}
    for l in range(2):
        # next layer's KQV of nano-batch 0 right after this layer's UGD of nano-batch 0,
        # ahead of this layer's O of nano-batch 1
        assert at[(l + 1) * n + K0] == at[l * n + U0] + 1
        assert at[(l + 1) * n + K0] < at[l * n + O1]
        assert at[(l + 1) * n + K1] == at[l * n + U1] + 1
    flat_at = {op: p for p, op in enumerate(flat)}
    assert all(flat_at[op] // n == op // n for op in flat)  # unpipelined: layer by layer
    # edges are the same either way
    e0, _, _ = abi.nf_stack_dependencies(hb, plan, 3, 0)
    e1, _, _ = abi.nf_stack_dependencies(hb, plan, 3, abi.NF_STACK_PIPELINE)
    assert sorted(e0) == sorted(e1)


def test_stack_rejects_bad_arguments(abi):
    b = sw.batch_from_lengths([5] * 4, [7], seed=0)
    hb = abi.HostBatch.from_batch(b)
    for n_layers, flags in ((0, 0), (2, 8)):
        with pytest.raises(abi.NanoflowError) as e:
            abi.nf_stack_dependencies(hb, None, n_layers, flags)
        assert e.value.status == abi.NF_E_ARG
