"""Host-side checks of libnanoflow (no GPU): exports, batch validation, slots, DAG."""

import json
import os
import re

import numpy as np
import pytest

from oracle import layer as ol
from synth import workloads as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_values.json")))


@pytest.fixture(scope="module")
def abi():
    from nano_intra_overlap_amd import abi as a

    a.load()
    return a


def test_library_exports_every_declared_function(abi):
    import ctypes

    declared = set()
    for name in os.listdir(os.path.join(ROOT, "include")):
        if name.endswith(".h"):
            text = open(os.path.join(ROOT, "include", name)).read()
            declared |= set(re.findall(r"^\s*(?:nf_status|void|const char \*)\s*\*?\s*(nf_\w+)\s*\(", text, re.M))
    # the calls the layer boundary is specified with, by name
    assert {"nf_ctx_create", "nf_ctx_destroy", "nf_last_error", "nf_layer_forward", "nf_op_gemm", "nf_op_rmsnorm",
            "nf_op_rope_kv_append", "nf_op_decode_attn", "nf_op_prefill_attn", "nf_profile_ops",
            "nf_profile_interference", "nf_plan_search"} <= declared
    lib = ctypes.CDLL(abi.LIB_PATH)
    missing = [n for n in sorted(declared) if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding calls nothing the header leaves undeclared
    bound = set(re.findall(r'^\s*"(nf_\w+)": \(', open(abi.__file__).read(), re.M))
    assert "nf_layer_forward" in bound
    undeclared = [n for n in sorted(bound) if n not in declared]
    assert not undeclared, undeclared
    assert abi.nf_version().startswith("nanoflow-mi355x")


def _cfg(abi, name="tiny"):
    return abi.make_cfg(sw.WORKLOADS[name].shape)


@pytest.mark.parametrize("seed", range(4))
def test_slots_bit_exact_against_oracle(abi, seed):
    rng = np.random.default_rng(seed)
    dec = rng.integers(0, 400, int(rng.integers(0, 30)))
    pre = rng.integers(1, 90, int(rng.integers(0, 4)))
    prefix = rng.integers(0, 50, pre.shape[0])
    if dec.size + pre.size == 0:
        dec = np.array([3])
    b = sw.batch_from_lengths(dec, pre, prefix, seed=seed)
    pos, slot = abi.nf_batch_slots(_cfg(abi), abi.HostBatch.from_batch(b), b.num_blocks)
    _, opos = ol.token_positions(b)
    oslot = [blk * 16 + off for blk, off in ol.new_token_slots(b, 16)]
    assert np.array_equal(pos, opos)
    assert np.array_equal(slot, np.asarray(oslot))


def test_slots_full_size_batch(abi):
    b = sw.make_batch("llama3_8b_layer", 0)
    pos, slot = abi.nf_batch_slots(_cfg(abi, "llama3_8b_layer"), abi.HostBatch.from_batch(b), b.num_blocks)
    oslot = [blk * 16 + off for blk, off in ol.new_token_slots(b, 16)]
    assert np.array_equal(slot, np.asarray(oslot))
    assert len(set(slot.tolist())) == b.n_tokens


def _status(abi, b, num_blocks, cfg=None, **over):
    hb = abi.HostBatch(over.get("dec", b.decode_ctx), over.get("pre", b.prefill_len), over.get("prefix", b.prefill_prefix),
                       over.get("bt", b.block_table))
    try:
        abi.nf_batch_slots(cfg or _cfg(abi), hb, num_blocks)
        return abi.NF_OK
    except abi.NanoflowError as e:
        return e.status


def test_batch_validation_error_codes(abi):
    b = sw.batch_from_lengths([20, 33], [17], [0], seed=1)
    assert _status(abi, b, b.num_blocks) == abi.NF_OK
    bt = b.block_table.copy()
    bt[1, 1] = b.num_blocks
    assert _status(abi, b, b.num_blocks, bt=bt) == abi.NF_E_BLOCK_RANGE
    bt = b.block_table.copy()
    bt[0, 0] = -1
    assert _status(abi, b, b.num_blocks, bt=bt) == abi.NF_E_BLOCK_RANGE
    assert _status(abi, b, b.num_blocks, bt=b.block_table[:, :1]) == abi.NF_E_BLOCK_TABLE_SHORT
    bt = b.block_table.copy()
    bt[1, 1] = bt[0, 1]  # request 1's new token lands in request 0's new-token block
    bt[1, 2] = bt[0, 1]
    assert _status(abi, b, b.num_blocks, bt=bt) in (abi.NF_E_SLOT_ALIAS, abi.NF_OK)
    dup = sw.batch_from_lengths([15, 15], [], seed=2)
    bt = dup.block_table.copy()
    bt[1, 0] = bt[0, 0]  # both decodes write position 15 of the same block
    assert _status(abi, dup, dup.num_blocks, bt=bt) == abi.NF_E_SLOT_ALIAS
    assert _status(abi, b, b.num_blocks, pre=[0]) == abi.NF_E_ARG
    assert _status(abi, b, b.num_blocks, dec=[-1, 3]) == abi.NF_E_ARG
    assert _status(abi, b, 0) == abi.NF_E_ARG
    bad = abi.make_cfg(sw.Shape(hidden=256, n_q=4, n_kv=2, head_dim=96, ffn=688))
    assert _status(abi, b, b.num_blocks, cfg=bad) == abi.NF_E_UNSUPPORTED
    bad = abi.make_cfg(sw.Shape(hidden=256, n_q=34, n_kv=2, head_dim=64, ffn=688))
    assert _status(abi, b, b.num_blocks, cfg=bad) == abi.NF_E_UNSUPPORTED


def test_moe_shape_validation(abi):
    import dataclasses

    b = sw.batch_from_lengths([20, 33], [17], [0], seed=1)
    moe = sw.WORKLOADS["tiny_moe"].shape
    assert _status(abi, b, b.num_blocks, cfg=abi.make_cfg(moe)) == abi.NF_OK
    assert _status(abi, b, b.num_blocks, cfg=abi.make_cfg(sw.WORKLOADS["mixtral_8x7b_layer"].shape)) == abi.NF_OK
    for bad in (dataclasses.replace(moe, n_experts=6), dataclasses.replace(moe, top_k=1),
                dataclasses.replace(moe, ffn=264), dataclasses.replace(moe, n_experts=32)):
        assert _status(abi, b, b.num_blocks, cfg=abi.make_cfg(bad)) == abi.NF_E_UNSUPPORTED, bad
    assert _status(abi, b, b.num_blocks, cfg=abi.make_cfg(dataclasses.replace(moe, n_experts=-1))) == abi.NF_E_ARG


def test_gemm_choice_is_always_an_available_variant(abi):
    """The library's own tile choice must be a configuration the launcher accepts for the
    shape and epilogue: every nano-batch row count of the workloads' projections (1..2048
    rows, each GEMM of the 8B, 70B-share, tiny and MoE shapes) and a sweep of other sizes."""
    variants = abi.nf_gemm_variants()
    shapes = set()
    for name in ("tiny", "llama3_8b_layer", "llama2_70b_tp8_layer", "tiny_moe", "mixtral_8x7b_layer"):
        sh = sw.WORKLOADS[name].shape
        q = sh.n_q * sh.head_dim
        shapes |= {(sh.qkv_rows, sh.hidden, 0), (sh.hidden, q, 1), (sh.ffn, sh.hidden, 2), (sh.hidden, sh.ffn, 1),
                   (sh.ffn, sh.hidden, 0)}
    shapes |= {(n, k, e) for n in (8, 64, 520, 1280, 4096, 6144, 8192) for k in (8, 96, 256, 4096) for e in (0, 1, 2)}
    for n, k, epi in sorted(shapes):
        for m in sorted({1, 7, 63, 64, 65, 127, 128, 200, 255, 256, 511, 512, 768, 1000, 1024, 1536, 2048, 4096}):
            v, ok = abi.nf_gemm_choice(m, n, k, epi)
            assert ok, (m, n, k, epi, v, variants[v])
    with pytest.raises(abi.NanoflowError):
        abi.nf_gemm_choice(16, 12, 64, 0)
    with pytest.raises(abi.NanoflowError):
        abi.nf_gemm_choice(16, 64, 64, 3)


def test_dependency_rule_pages_example(abi):
    """O1 on tokens 0-767 depends on Attn1 (0-767) but not on Attn2 (768-2048)."""
    ex = GOLDEN["intersection_dependency_example"]
    b = sw.batch_from_lengths(np.full(2048, 10), [], seed=0)
    hb = abi.HostBatch.from_batch(b)
    bounds = [0, ex["attn1"][1], ex["attn2"][1]]
    plan = abi.HostPlan(bounds, [(k, j, 0) for k in range(5) for j in range(2)], 1)
    edges, order = abi.nf_plan_dependencies(hb, plan)
    idx = {(k, j): i for i, (k, j, _) in enumerate(plan.ops)}
    e = set(edges)
    o1, attn1, attn2 = idx[(abi.NF_OP_O, 0)], idx[(abi.NF_OP_DECATTN, 0)], idx[(abi.NF_OP_DECATTN, 1)]
    assert ((attn1, o1) in e) == ex["o1_depends_on_attn1"]
    assert ((attn2, o1) in e) == ex["o1_depends_on_attn2"]


def test_dependencies_match_oracle_rule(abi):
    from oracle import schedule as osch

    rng = np.random.default_rng(3)
    for trial in range(20):
        dec = rng.integers(0, 100, int(rng.integers(0, 40)))
        pre = rng.integers(1, 60, int(rng.integers(0, 4)))
        if dec.size + pre.size == 0:
            pre = np.array([5])
        b = sw.batch_from_lengths(dec, pre, None, seed=trial)
        T = b.n_tokens
        n = int(rng.integers(1, min(5, T) + 1))
        cuts = sorted(rng.choice(np.arange(1, T), size=n - 1, replace=False).tolist()) if n > 1 else []
        bounds = [0] + cuts + [T]
        ops = [(k, j, 0) for k in range(5) for j in range(n)]  # kind-major: always a valid order
        plan = abi.HostPlan(bounds, ops, 1)
        edges, _ = abi.nf_plan_dependencies(abi.HostBatch.from_batch(b), plan)
        got = {(ops[i][:2], ops[j][:2]) for i, j in edges}
        want = osch.dependencies(b, bounds)
        assert got == want, (trial, bounds)


def test_plan_order_deadlock_is_rejected(abi):
    b = sw.batch_from_lengths([5] * 10, [20], seed=0)
    T = b.n_tokens
    # one stream listing O before the decode attention it depends on
    ops = [(abi.NF_OP_KQV, 0, 0), (abi.NF_OP_O, 0, 0), (abi.NF_OP_DECATTN, 0, 0), (abi.NF_OP_PFATTN, 0, 0),
           (abi.NF_OP_UGD, 0, 0)]
    with pytest.raises(abi.NanoflowError) as e:
        abi.nf_plan_dependencies(abi.HostBatch.from_batch(b), abi.HostPlan([0, T], ops, 1))
    assert e.value.status == abi.NF_E_PLAN
    for bounds in ([0, T - 1], [0, 5, 5, T], [1, T]):
        n = len(bounds) - 1
        with pytest.raises(abi.NanoflowError):
            abi.nf_plan_dependencies(abi.HostBatch.from_batch(b),
                                     abi.HostPlan(bounds, [(k, j, 0) for k in range(5) for j in range(n)], 1))


def test_plan_templates_never_deadlock(abi):
    from nano_intra_overlap_amd import plans

    rng = np.random.default_rng(11)
    for trial in range(25):
        dec = rng.integers(0, 50, int(rng.integers(0, 30)))
        pre = rng.integers(1, 70, int(rng.integers(1, 4)))
        b = sw.batch_from_lengths(dec, pre, None, seed=trial)
        hb = abi.HostBatch.from_batch(b)
        T = b.n_tokens
        n = int(rng.integers(1, min(5, T) + 1))
        bounds = [0] + sorted(rng.choice(np.arange(1, T), size=n - 1, replace=False).tolist()) + [T]
        for plan in (plans.sequential(hb, bounds), plans.overlap(hb, bounds),
                     plans.overlap(hb, bounds, prefill_on_memory=False),
                     plans.overlap(hb, bounds, memory_kinds=(abi.NF_OP_O,))):
            abi.nf_plan_dependencies(hb, plan)  # raises NF_E_PLAN on a deadlocking order


def test_overlap_memory_kinds_places_o_after_its_attention(abi):
    """memory_kinds=(O,): every O runs on the memory stream, after its nano-batch's
    attention there; the compute stream keeps KQV and Up/Gate/Down."""
    from nano_intra_overlap_amd import plans

    b = sw.make_batch("tiny", 0)
    hb = abi.HostBatch.from_batch(b)
    bounds = [0, 39, b.n_tokens]
    plan = plans.overlap(hb, bounds, memory_kinds=(abi.NF_OP_O,))
    ops = plan.ops
    on_memory = [(k, j) for k, j, s in ops if s == 1]
    assert {k for k, _ in on_memory} <= {abi.NF_OP_DECATTN, abi.NF_OP_PFATTN, abi.NF_OP_O}
    assert all(s == 0 for k, _, s in ops if k in (abi.NF_OP_KQV, abi.NF_OP_UGD))
    for j in range(len(bounds) - 1):
        assert on_memory.index((abi.NF_OP_O, j)) > on_memory.index((abi.NF_OP_DECATTN, j))
    abi.nf_plan_dependencies(hb, plan)
    with pytest.raises(ValueError):
        plans.overlap(hb, bounds, unmasked_kinds=(abi.NF_OP_UGD,), memory_kinds=(abi.NF_OP_O,))


def test_cu_mask_helper_balances_xcds(abi):
    for frac in (0.125, 0.25, 0.5, 0.75, 1.0):
        m = abi.cu_mask(frac)
        bits = [(m[i // 32] >> (i % 32)) & 1 for i in range(256)]
        per = [sum(bits[i] for i in range(256) if i % 8 == x) for x in range(8)]
        assert len(set(per)) == 1 and per[0] == round(frac * 32)
