"""Layer calls issued back to back on one context, with no host synchronisation between them.

Every call packs its batch metadata (positions, slots, work lists, block table) into the
context's pinned staging and copies it to the device ahead of its kernels; the staging is
reused only after the previous copy from it is done, and the device copy is rewritten in
stream order after the previous call's kernels. These tests alternate two different batches
call after call (and plans with one stream and with two, and stand-alone attention calls)
and check every call's output against the oracle.

The two batches have the same request counts and prefill lengths, different decode context
lengths, and share one block table whose rows are filled with distinct valid block ids to
their full width: their metadata has the same layout, and every value in either batch's
metadata addresses memory inside the buffers of both.
"""

import numpy as np
import pytest

from oracle import layer as ol
from synth import workloads as sw
from tests.gpu_util import TOL, f64, log_case, rand_bf16, rel_inf

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    from nano_intra_overlap_amd import abi

    c = abi.nf_ctx_create(0)
    yield c
    abi.nf_ctx_destroy(c)


def _twin_batches():
    """Two tiny batches with one shared, fully populated block table."""
    base = sw.make_batch("tiny", 0)
    rng = np.random.default_rng(11)
    ctx_a = base.decode_ctx.astype(np.int32)
    ctx_b = rng.integers(16, 129, size=ctx_a.shape[0]).astype(np.int32)
    assert not np.array_equal(ctx_a, ctx_b)
    pre = base.prefill_len.astype(np.int32)
    need = np.concatenate([np.maximum(ctx_a, ctx_b) + 1, pre])
    max_blocks = int((need.max() + 15) // 16)
    n_req = need.shape[0]
    num_blocks = n_req * max_blocks + 4
    table = rng.permutation(num_blocks)[: n_req * max_blocks].astype(np.int32).reshape(n_req, max_blocks)
    zeros = np.zeros_like(pre)
    a = sw.Batch(ctx_a, pre, zeros, table.copy(), num_blocks)
    b = sw.Batch(ctx_b, pre, zeros.copy(), table.copy(), num_blocks)
    return a, b


def test_back_to_back_calls_alternate_batches(ctx):
    from nano_intra_overlap_amd import abi, plans
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_bits, bf16_tensor

    wl = sw.WORKLOADS["tiny"]
    shape = wl.shape
    batches = _twin_batches()
    w = sw.make_weights(shape, 3, gain_jitter=0.1)
    wd = DeviceWeights(w, "cuda")
    cfg = abi.make_cfg(shape)
    stream = torch.cuda.current_stream().cuda_stream
    cases = []
    for i, b in enumerate(batches):
        x = sw.make_x(shape, b.n_tokens, 20 + i)
        kp, vp = sw.make_kv_pool(shape, b.num_blocks, 30 + i)
        ref = ol.layer_forward(shape, w, x, b, kp, vp)
        hb = abi.HostBatch.from_batch(b)
        cases.append(dict(b=b, kp=kp, vp=vp, ref=ref, hb=hb, x=bf16_tensor(x, "cuda"),
                          pool=DevicePool.from_host(kp, vp, "cuda"),
                          plans=[None, plans.overlap(hb, [0, 39, b.n_tokens])]))
    torch.cuda.synchronize()
    order = [(0, 0), (1, 1), (0, 1), (1, 0), (0, 0), (1, 1), (0, 1), (1, 0)]  # (batch, plan)
    ys = []
    log_case(f"tiny twin batches, {len(order)} layer calls back to back, no host sync")
    for i, p in order:
        c = cases[i]
        y = torch.full_like(c["x"], float("nan"))
        abi.nf_layer_forward(ctx, cfg, wd.desc, c["x"].data_ptr(), y.data_ptr(), c["hb"], c["pool"].desc,
                             c["plans"][p], stream)
        ys.append(y)
    torch.cuda.synchronize()
    for (i, p), y in zip(order, ys):
        e = rel_inf(f64(bf16_bits(y)), cases[i]["ref"]["y"])
        assert e <= TOL, (i, p, e)
    # repeated calls rewrite this iteration's slots with the same values: each pool holds
    # its oracle's written K/V there and its initial contents everywhere else
    for c in cases:
        b = c["b"]
        kg, vg = c["pool"].host_bits()
        new = np.zeros((b.num_blocks, 16), bool)
        for blk, off in ol.new_token_slots(b, 16):
            new[blk, off] = True
        assert np.array_equal(kg.transpose(0, 3, 1, 2, 4)[~new], c["kp"].transpose(0, 3, 1, 2, 4)[~new])
        assert np.array_equal(vg.transpose(0, 3, 1, 2)[~new], c["vp"].transpose(0, 3, 1, 2)[~new])
        kr, vr = c["ref"]["k_pool"], c["ref"]["v_pool"]
        assert rel_inf(f64(kg.transpose(0, 3, 1, 2, 4)[new]), f64(kr.transpose(0, 3, 1, 2, 4)[new])) <= TOL
        assert rel_inf(f64(vg.transpose(0, 3, 1, 2)[new]), f64(vr.transpose(0, 3, 1, 2)[new])) <= TOL


def test_back_to_back_per_op_and_layer_calls(ctx):
    """Stand-alone decode-attention calls of one batch interleaved with layer calls of the
    other, no host sync: every output against the oracle."""
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_bits, bf16_tensor

    wl = sw.WORKLOADS["tiny"]
    shape = wl.shape
    a, b = _twin_batches()
    w = sw.make_weights(shape, 4)
    wd = DeviceWeights(w, "cuda")
    cfg = abi.make_cfg(shape)
    stream = torch.cuda.current_stream().cuda_stream
    # batch a: layer calls
    x_a = sw.make_x(shape, a.n_tokens, 40)
    kpa, vpa = sw.make_kv_pool(shape, a.num_blocks, 41)
    ref_a = ol.layer_forward(shape, w, x_a, a, kpa, vpa)
    xa = bf16_tensor(x_a, "cuda")
    pool_a = DevicePool.from_host(kpa, vpa, "cuda")
    hba = abi.HostBatch.from_batch(a)
    # batch b: decode attention alone (q from a qkv buffer, every key from the pool)
    rng = np.random.default_rng(44)
    qkv = rand_bf16(rng, (b.n_tokens, shape.qkv_rows), 1.3)
    kpb, vpb = sw.make_kv_pool(shape, b.num_blocks, 43)
    n_q, d = shape.n_q, shape.head_dim
    q = f64(qkv[:, : n_q * d]).reshape(b.n_tokens, n_q, d)
    ref_b = ol.attention_all(shape, b, q, kpb, vpb).reshape(b.n_tokens, n_q * d)
    pool_b = DevicePool.from_host(kpb, vpb, "cuda")
    dqkv = bf16_tensor(qkv, "cuda")
    hbb = abi.HostBatch.from_batch(b)
    torch.cuda.synchronize()
    ys, outs = [], []
    log_case("tiny twin batches: layer calls and decode-attention calls back to back")
    for _ in range(3):
        y = torch.full_like(xa, float("nan"))
        abi.nf_layer_forward(ctx, cfg, wd.desc, xa.data_ptr(), y.data_ptr(), hba, pool_a.desc, None, stream)
        ys.append(y)
        o = torch.full((b.n_tokens, n_q * d), float("nan"), dtype=torch.bfloat16, device="cuda")
        abi.nf_op_decode_attn(ctx, cfg, dqkv.data_ptr(), hbb, pool_b.desc, o.data_ptr(), 0, stream)
        outs.append(o)
    torch.cuda.synchronize()
    for y in ys:
        assert rel_inf(f64(bf16_bits(y)), ref_a["y"]) <= TOL
    n_dec = b.n_decode
    for o in outs:
        assert rel_inf(f64(bf16_bits(o))[:n_dec], ref_b[:n_dec]) <= TOL
