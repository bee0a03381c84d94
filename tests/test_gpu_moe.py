"""Mixture-of-experts FFN and MoE layer parity against the CPU oracle, through the C ABI.

Routing is a decision taken on floating point: the GPU ranks fp32 logits, the oracle
float64 ones, and the two h2 inputs of a whole layer may differ in a last bf16 bit. A token
whose second and third router logits (oracle) lie within ROUTE_MARGIN of each other may
legitimately be routed either way; for such tokens the test checks that the GPU's choice is
a valid one (its logits are within the margin of the oracle's choice) and leaves their rows
out of the value comparison. Every other token must pick exactly the oracle's two experts,
with the same weights, and match the oracle's output row.

* the MoE FFN alone (nf_op_moe_ffn) on the tiny MoE shape: 1, 7, 78 and 1000 tokens (one
  token leaves six experts empty; 1000 tokens fill 256-row tiles), every grouped tile
  variant, and a skewed router (one expert takes most tokens);
* the tiny MoE layer under the null, 2-nano-batch sequential and overlap plans;
* the Mixtral-8x7B-shaped layer at the full 2048-token batch (overlap plan), sampled.
"""

import numpy as np
import pytest

from oracle import layer as ol
from synth import workloads as sw
from tests.gpu_util import TOL, f64, log_case, rand_bf16, rel_inf

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ROUTE_MARGIN_OP = 1e-4     # same bf16 h2 on both sides: only the dot products' rounding differs
ROUTE_MARGIN_LAYER = 5e-3  # h2 from each side's own layer: a last-bit difference of h2 moves logits


@pytest.fixture(scope="module")
def ctx():
    from nano_intra_overlap_amd import abi

    c = abi.nf_ctx_create(0)
    yield c
    abi.nf_ctx_destroy(c)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ambiguous(logits, margin):
    srt = -np.sort(-logits, axis=1)
    return (srt[:, 1] - srt[:, 2]) < margin


def check_routing(logits, ref_sel, ref_wts, sel, wts, margin):
    """Unambiguous tokens: the same two experts with the same weights (the order of the two
    may differ only when their logits tie within the margin). Ambiguous tokens: a valid
    choice. Returns the mask of unambiguous tokens."""
    amb = _ambiguous(logits, margin)
    for t in range(logits.shape[0]):
        got = dict(zip(sel[t].tolist(), wts[t].tolist()))
        if not amb[t]:
            want = dict(zip(ref_sel[t].tolist(), ref_wts[t].tolist()))
            assert set(got) == set(want), (t, got, want)
            for e in want:
                assert abs(got[e] - want[e]) <= 1e-4, (t, e, got[e], want[e])
        else:
            assert len(got) == 2 and all(0 <= e < logits.shape[1] for e in got)
            third = -np.sort(-logits[t])[2]
            assert all(logits[t, e] >= third - margin for e in got), t
        assert abs(sum(got.values()) - 1.0) <= 1e-5
    return ~amb


def _moe_op_case(ctx, shape, w, dw, T, seed, variants=(-1, -1), h2_shift=0.0):
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import bf16_bits, bf16_tensor

    rng = np.random.default_rng(seed)
    h2 = sw.f32_to_bf16_bits(sw.bf16_bits_to_f32(rand_bf16(rng, (T, shape.hidden))) + np.float32(h2_shift))
    x1 = rand_bf16(rng, (T, shape.hidden))
    h2_d, x1_d = bf16_tensor(h2, "cuda"), bf16_tensor(x1, "cuda")
    y_d = torch.full_like(x1_d, float("nan"))
    sel_d = torch.full((T, 2), -1, dtype=torch.int32, device="cuda")
    wts_d = torch.full((T, 2), float("nan"), dtype=torch.float32, device="cuda")
    for which, v in enumerate(variants):
        abi.nf_ctx_set_gemm_variant(ctx, abi.NF_OP_UGD, which, v)
    log_case(f"moe ffn op T={T} seed={seed} variants={variants}")
    abi.nf_op_moe_ffn(ctx, abi.make_cfg(shape), dw.desc, h2_d.data_ptr(), x1_d.data_ptr(), y_d.data_ptr(), T,
                      sel_d.data_ptr(), wts_d.data_ptr(), _stream())
    torch.cuda.synchronize()
    for which in (0, 1):
        abi.nf_ctx_set_gemm_variant(ctx, abi.NF_OP_UGD, which, -1)
    W = {k: ol.bf16_to_f64(v) for k, v in w.items()}
    ffn, sel, wts, logits = ol.moe_ffn(f64(h2), W, shape, ol.store_bf16)
    ref_y = ol.store_bf16(f64(x1) + ffn)
    ok = check_routing(logits, sel, wts, sel_d.cpu().numpy(), wts_d.cpu().numpy(), ROUTE_MARGIN_OP)
    y = f64(bf16_bits(y_d))
    assert np.isfinite(y).all()
    assert rel_inf(y[ok], ref_y[ok]) <= TOL, rel_inf(y[ok], ref_y[ok])
    return sel


@pytest.mark.parametrize("T", [1, 7, 78, 1000])
def test_moe_ffn_op_tiny(ctx, T):
    from nano_intra_overlap_amd.device import DeviceWeights

    shape = sw.WORKLOADS["tiny_moe"].shape
    w = sw.make_weights(shape, 3)
    sel = _moe_op_case(ctx, shape, w, DeviceWeights(w, "cuda"), T, seed=T)
    if T == 1:
        assert len(set(sel[0].tolist())) == 2  # six experts without a row


def test_moe_ffn_op_every_grouped_variant(ctx):
    from nano_intra_overlap_amd.device import DeviceWeights

    shape = sw.WORKLOADS["tiny_moe"].shape
    w = sw.make_weights(shape, 4)
    dw = DeviceWeights(w, "cuda")
    for ug, down in ((6, 7), (7, 6), (8, 9), (9, 8), (12, 13), (12, 18), (22, 28), (28, 22), (29, 30), (30, 29),
                     (21, 24), (24, 21)):
        _moe_op_case(ctx, shape, w, dw, 300, seed=ug, variants=(ug, down))


def test_moe_ffn_op_skewed_router(ctx):
    """One expert's router row aligned with a component every h2 row shares: nearly every
    token picks it, the other experts share the second choices."""
    from nano_intra_overlap_amd.device import DeviceWeights

    shape = sw.WORKLOADS["tiny_moe"].shape
    w = sw.make_weights(shape, 5)
    r = sw.bf16_bits_to_f32(w["w_router"])
    r[2] = np.abs(r[2])
    w["w_router"] = sw.f32_to_bf16_bits(r)
    sel = _moe_op_case(ctx, shape, w, DeviceWeights(w, "cuda"), 600, seed=6, h2_shift=0.5)
    counts = np.bincount(sel.ravel(), minlength=shape.n_experts)
    assert counts[2] > 0.3 * sel.size, counts


# ----------------------------------------------------------------------------- the layer


def _check_moe_layer(ctx, shape, b, kp, vp, ref, y_dev, pool, margin, rows=None):
    from nano_intra_overlap_amd.device import bf16_bits
    from tests.test_gpu_layer import _attn_buffer

    y = f64(bf16_bits(y_dev))
    assert np.isfinite(y).all()
    if rows is not None:
        y = y[rows]
    amb = _ambiguous(ref["moe_logits"], margin)
    print(f"  ambiguous routing: {int(amb.sum())} of {amb.size} tokens", flush=True)
    assert rel_inf(y[~amb], ref["y"][~amb]) <= TOL, rel_inf(y[~amb], ref["y"][~amb])
    attn = f64(_attn_buffer(ctx, b.n_tokens, shape.n_q * shape.head_dim))
    if rows is not None:
        attn = attn[rows]
    assert rel_inf(attn, ref["attn"]) <= TOL
    if pool is not None:
        kg, vg = pool.host_bits()
        new = np.zeros((b.num_blocks, 16), bool)
        for blk, off in ol.new_token_slots(b, 16):
            new[blk, off] = True
        assert np.array_equal(kg.transpose(0, 3, 1, 2, 4)[~new], kp.transpose(0, 3, 1, 2, 4)[~new])
        assert np.array_equal(vg.transpose(0, 3, 1, 2)[~new], vp.transpose(0, 3, 1, 2)[~new])
        assert rel_inf(f64(kg.transpose(0, 3, 1, 2, 4)[new]), f64(ref["k_pool"].transpose(0, 3, 1, 2, 4)[new])) <= TOL


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_moe_layer_plans(ctx, seed):
    from nano_intra_overlap_amd import abi, plans
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_tensor

    wl = sw.WORKLOADS["tiny_moe"]
    shape = wl.shape
    b = sw.make_batch("tiny_moe", seed)
    w = sw.make_weights(shape, seed, gain_jitter=0.1)
    x = sw.make_x(shape, b.n_tokens, seed)
    kp, vp = sw.make_kv_pool(shape, b.num_blocks, seed)
    ref = ol.layer_forward(shape, w, x, b, kp, vp)
    dw, xd = DeviceWeights(w, "cuda"), bf16_tensor(x, "cuda")
    hb = abi.HostBatch.from_batch(b)
    T = b.n_tokens
    for name, plan in (("null", None), ("seq2", plans.sequential(hb, [0, 39, T])),
                       ("overlap2", plans.overlap(hb, [0, 39, T])),
                       ("overlap4", plans.overlap(hb, [0, 10, 20, 50, T], prefill_on_memory=False))):
        pool = DevicePool.from_host(kp, vp, "cuda")
        y = torch.full_like(xd, float("nan"))
        log_case(f"tiny moe layer seed={seed} plan={name}")
        abi.nf_layer_forward(ctx, abi.make_cfg(shape), dw.desc, xd.data_ptr(), y.data_ptr(), hb, pool.desc, plan,
                             _stream())
        torch.cuda.synchronize()
        _check_moe_layer(ctx, shape, b, kp, vp, ref, y, pool, ROUTE_MARGIN_LAYER)


def test_full_size_moe_layer_sampled(ctx):
    """Mixtral-8x7B-shaped layer, 2048-token batch, overlap plan; the weights come from the
    counter-based generator on the device and are copied to the host for the oracle."""
    from nano_intra_overlap_amd import abi, plans
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_tensor
    from synth.workloads import make_kv_pool_torch

    name, seed = "mixtral_8x7b_layer", 0
    shape = sw.WORKLOADS[name].shape
    b = sw.make_batch(name, seed)
    dw = DeviceWeights.from_int16(sw.make_weights_counter_torch(shape, seed, 0, device="cuda"))
    w = dw.host_bits()
    x = sw.make_x(shape, b.n_tokens, seed)
    pool = DevicePool.from_int16(*make_kv_pool_torch(shape, b.num_blocks, seed, device="cuda"))
    xd = bf16_tensor(x, "cuda")
    y = torch.full_like(xd, float("nan"))
    hb = abi.HostBatch.from_batch(b)
    plan = plans.overlap(hb, plans.even_bounds(b.n_tokens, 2))
    log_case(f"full-size moe layer {name} seed={seed} overlap2")
    abi.nf_layer_forward(ctx, abi.make_cfg(shape), dw.desc, xd.data_ptr(), y.data_ptr(), hb, pool.desc, plan,
                         _stream())
    torch.cuda.synchronize()
    from tests.gpu_util import oracle_subbatch

    rng = np.random.default_rng(seed + 99)
    sample = sorted(rng.choice(b.n_decode, size=24, replace=False).tolist()) + list(range(b.n_decode, b.n_requests))
    rows, used, compact, ref = oracle_subbatch(shape, b, w, x, sample, seed)
    _check_moe_layer(ctx, shape, b, None, None, ref, y, None, ROUTE_MARGIN_LAYER, rows=rows)
