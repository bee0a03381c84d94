"""Per-operation parity of the HIP kernels against the CPU oracle, through the C ABI.

Inputs are seeded; shapes span several tiles and ragged tails. Tolerance: max relative
error 1e-2 per output tensor (bf16 storage, fp32 accumulation); KV slots bit-exact.
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


def _dev(bits):
    from nano_intra_overlap_amd.device import bf16_tensor

    return bf16_tensor(bits, "cuda")


def _host(t):
    from nano_intra_overlap_amd.device import bf16_bits

    return bf16_bits(t)


GEMM_SHAPES = [(1, 64, 64), (77, 520, 264), (300, 688, 688), (513, 1024, 256), (2048, 640, 512), (77, 520, 256),
               (300, 688, 672), (1, 256, 96)]
# the layer's shapes (K, N of each projection at the 8B and 70B-share sizes), checked on sampled rows
LAYER_GEMMS = [(1024, 6144, 4096, 0), (2048, 4096, 4096, 1), (1536, 14336, 4096, 2), (1024, 4096, 14336, 1),
               (2048, 1280, 8192, 0), (1024, 1280, 8192, 0), (512, 3584, 8192, 2), (2048, 8192, 3584, 1),
               (1024, 8192, 1024, 1)]


def _supported(v, k, epi, bn, ks=1, waves=4, bk=32):
    # split-K slices are whole slabs (sizes differing by at most one): at least one per slice
    return (not (epi == 2 and (bn < 128 or (bn // (waves // 2)) % 64)) and not (v >= 6 and k % bk)
            and not (ks > 1 and (epi == 2 or k // bk < ks)))


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_gemm_all_variants(ctx, m, n, k, epi):
    from nano_intra_overlap_amd import abi

    rng = np.random.default_rng(m * 31 + n * 7 + k + epi)
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (2 * n if epi == 2 else n, k), 0.05)
    R = rand_bf16(rng, (m, n))
    ref = ol.linear(f64(A), f64(B))
    if epi == 1:
        ref = f64(R) + ref
    if epi == 2:
        ref = ol.swiglu(ref, n)
    dA, dB, dR = _dev(A), _dev(B), _dev(R)
    for v, (bm, bn, bk, ks, waves) in enumerate(abi.nf_gemm_variants()):
        if not _supported(v, k, epi, bn, ks, waves, bk):
            continue
        dC = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        log_case(f"gemm m={m} n={n} k={k} epi={epi} variant={v}")
        abi.nf_op_gemm(ctx, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), dR.data_ptr(), m, n, k, epi, v,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got = f64(_host(dC))
        assert np.isfinite(got).all(), f"variant {v}: unwritten outputs"
        err = rel_inf(got, ref)
        assert err <= TOL, f"variant {v} ({bm}x{bn}x{bk}, {ks} K slices): rel err {err}"


@pytest.mark.parametrize("m,n,k,epi", LAYER_GEMMS)
def test_gemm_layer_shapes_sampled_rows(ctx, m, n, k, epi):
    from nano_intra_overlap_amd import abi

    rng = np.random.default_rng(m + n + k + epi)
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (2 * n if epi == 2 else n, k), 0.02)
    R = rand_bf16(rng, (m, n))
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 40, replace=False)]))
    ref = ol.linear(f64(A[rows]), f64(B))
    if epi == 1:
        ref = f64(R[rows]) + ref
    if epi == 2:
        ref = ol.swiglu(ref, n)
    dA, dB, dR = _dev(A), _dev(B), _dev(R)
    for v, (bm, bn, bk, ks, waves) in [(-1, (0, 0, 0, 1, 4))] + list(enumerate(abi.nf_gemm_variants())):
        if v >= 0 and (not _supported(v, k, epi, bn, ks, waves, bk) or v < 6):
            continue
        dC = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        log_case(f"gemm layer shape m={m} n={n} k={k} epi={epi} variant={v}")
        abi.nf_op_gemm(ctx, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), dR.data_ptr(), m, n, k, epi, v,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        full = _host(dC)
        assert not np.isnan(f64(full)).any(), f"variant {v}: unwritten outputs"
        err = rel_inf(f64(full[rows]), ref)
        assert err <= TOL, f"variant {v}: rel err {err}"


@pytest.mark.parametrize("m,n,k,epi", [(2048, 14336, 4096, 2), (300, 16640, 96, 2), (512, 33280, 64, 0),
                                        (512, 33280, 64, 1), (256, 2048, 64, 2)])
def test_gemm_balanced_last_round(ctx, m, n, k, epi):
    """Variants 19, 26 and 35 (64-deep; 35 with 4 waves) split the columns between a 256x256 launch and a last
    round of half tiles (at these shapes the last round of 256x256 tiles would be at most half full; the
    last shape has fewer tiles than CUs and takes the plain launch). Each output element
    sums k in the same order in every tile shape: bit-identical to variant 12, and the
    oracle's values on sampled rows."""
    from nano_intra_overlap_amd import abi

    rng = np.random.default_rng(m + n + epi)
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (2 * n if epi == 2 else n, k), 0.05)
    R = rand_bf16(rng, (m, n))
    dA, dB, dR = _dev(A), _dev(B), _dev(R)
    outs = {}
    for v in (12, 19) + ((26, 35) if k % 64 == 0 else ()):
        dC = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        log_case(f"gemm balanced m={m} n={n} k={k} epi={epi} variant={v}")
        abi.nf_op_gemm(ctx, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), dR.data_ptr(), m, n, k, epi, v,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        outs[v] = _host(dC)
    for v in outs:
        assert np.array_equal(outs[v], outs[12]), f"variant {v} differs from variant 12"
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 24, replace=False)]))
    ref = ol.linear(f64(A[rows]), f64(B))
    if epi == 1:
        ref = f64(R[rows]) + ref
    if epi == 2:
        ref = ol.swiglu(ref, n)
    got = f64(outs[19])
    assert np.isfinite(got).all()
    assert rel_inf(got[rows], ref) <= TOL


@pytest.mark.parametrize("m,n,k,epi", [(600, 1000, 1024, 0), (600, 1000, 1024, 1), (513, 768, 640, 2), (64, 256, 64, 1),
                                       (300, 512, 128, 0), (300, 512, 192, 1), (257, 1024, 256, 2)])
def test_gemm_deep_slabs_bit_identical(ctx, m, n, k, epi):
    """The 64-deep slab variants (21-24, 26-30, 35, and 32-34 with the B operand in its own
    ring of 3 slabs) sum k in the same order as the 32-deep ones: every output bit-identical to
    variant 12 (ragged m and n; 1, 2, 3 and 4 slabs of 64, which take every branch of the
    split ring's prologue and drain)."""
    from nano_intra_overlap_amd import abi

    rng = np.random.default_rng(m + 3 * n + k + epi)
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (2 * n if epi == 2 else n, k), 0.05)
    R = rand_bf16(rng, (m, n))
    dA, dB, dR = _dev(A), _dev(B), _dev(R)
    outs = {}
    for v in (12, 21, 22, 23, 24, 26, 27, 28, 29, 30, 32, 33, 34, 35):
        if v in (23, 27) and epi == 2:
            continue
        dC = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        log_case(f"gemm deep slabs m={m} n={n} k={k} epi={epi} variant={v}")
        abi.nf_op_gemm(ctx, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), dR.data_ptr(), m, n, k, epi, v,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        outs[v] = _host(dC)
    for v, o in outs.items():
        assert np.array_equal(o, outs[12]), f"variant {v} differs from variant 12"
    ref = ol.linear(f64(A), f64(B))
    if epi == 1:
        ref = f64(R) + ref
    if epi == 2:
        ref = ol.swiglu(ref, n)
    assert rel_inf(f64(outs[12]), ref) <= TOL


@pytest.mark.parametrize("variant", [-1, 6, 7, 9, 10, 11, 12, 13, 14, 15, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30,
                                     31, 32, 33, 34, 35, 36, 37, 38, 39, 40])
def test_gemm_residual_in_place(ctx, variant):
    from nano_intra_overlap_amd import abi

    rng = np.random.default_rng(5 + variant)
    m, n, k = 200, 256, 256
    A, B, R = rand_bf16(rng, (m, k)), rand_bf16(rng, (n, k), 0.05), rand_bf16(rng, (m, n))
    ref = f64(R) + ol.linear(f64(A), f64(B))
    dA, dB, dR = _dev(A), _dev(B), _dev(R)  # keep every operand alive until the kernel ran
    log_case(f"gemm residual aliasing C=R variant={variant}")
    abi.nf_op_gemm(ctx, dA.data_ptr(), dB.data_ptr(), dR.data_ptr(), dR.data_ptr(), m, n, k, 1, variant,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rel_inf(f64(_host(dR)), ref) <= TOL


@pytest.mark.parametrize("m,n", [(1, 256), (78, 4096), (33, 8192), (5, 688)])
def test_rmsnorm(ctx, m, n):
    from nano_intra_overlap_amd import abi

    rng = np.random.default_rng(m + n)
    x = rand_bf16(rng, (m, n), 2.0)
    g = sw.f32_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(n).astype(np.float32))
    ref = ol.rmsnorm(f64(x), f64(g), 1e-5)
    dout = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    dx, dg = _dev(x), _dev(g)
    log_case(f"rmsnorm m={m} n={n}")
    abi.nf_op_rmsnorm(ctx, dx.data_ptr(), dg.data_ptr(), dout.data_ptr(), m, n, 1e-5,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rel_inf(f64(_host(dout)), ref) <= TOL


CANARY = 0x7FC1  # NaN pattern never produced by rounding finite values


def _shape(n_q, n_kv, d, H=256):
    return sw.Shape(hidden=H, n_q=n_q, n_kv=n_kv, head_dim=d, ffn=H)


@pytest.mark.parametrize("n_q,n_kv,d", [(4, 2, 64), (32, 8, 128), (8, 1, 128)])
def test_rope_kv_append_slots_bit_exact(ctx, n_q, n_kv, d):
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool

    shape = _shape(n_q, n_kv, d)
    rng = np.random.default_rng(n_q + d)
    b = sw.batch_from_lengths(rng.integers(0, 300, 23), [37, 1, 16], [0, 5, 40], seed=3, spare_blocks=6)
    T = b.n_tokens
    qkv = rand_bf16(rng, (T, shape.qkv_rows), 1.3)
    kp = np.full((b.num_blocks, n_kv, d // 32, 16, 32), CANARY, np.uint16)
    vp = np.full((b.num_blocks, n_kv, d, 16), CANARY, np.uint16)
    _, pos = ol.token_positions(b)
    q = ol.rope(f64(qkv[:, : n_q * d]).reshape(T, n_q, d), pos, shape.rope_base)
    k = ol.rope(f64(qkv[:, n_q * d : (n_q + n_kv) * d]).reshape(T, n_kv, d), pos, shape.rope_base)
    v = f64(qkv[:, (n_q + n_kv) * d :]).reshape(T, n_kv, d)
    k_ref, v_ref = ol.write_kv(kp, vp, b, 16, k, v)

    dqkv = _dev(qkv)
    pool = DevicePool.from_host(kp, vp, "cuda")
    hb = abi.HostBatch.from_batch(b)
    log_case(f"rope_kv n_q={n_q} n_kv={n_kv} d={d}")
    abi.nf_op_rope_kv_append(ctx, abi.make_cfg(shape), dqkv.data_ptr(), hb, pool.desc,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    kg, vg = pool.host_bits()
    # the set of written slots is exactly the oracle's
    wk = kg != CANARY
    wv = vg != CANARY
    assert np.array_equal(wk, k_ref != CANARY)
    assert np.array_equal(wv, v_ref != CANARY)
    # values: V is copied (bit-exact); K and q within tolerance
    assert np.array_equal(vg, v_ref)
    assert rel_inf(f64(kg[wk]), f64(k_ref[wk])) <= TOL
    qg = f64(_host(dqkv)[:, : n_q * d]).reshape(T, n_q, d)
    assert rel_inf(qg, q) <= TOL
    # k is rotated in place too (the same bf16 values the pool received); v columns are left
    # as they were
    kq = _host(dqkv)[:, n_q * d : (n_q + n_kv) * d]
    assert rel_inf(f64(kq).reshape(T, n_kv, d), k) <= TOL
    kq_pool = ol.write_kv(np.full_like(kp, CANARY), np.full_like(vp, CANARY), b, 16,
                          f64(kq).reshape(T, n_kv, d), v)[0]
    assert np.array_equal(kg[wk], kq_pool[wk])
    assert np.array_equal(_host(dqkv)[:, (n_q + n_kv) * d :], qkv[:, (n_q + n_kv) * d :])


def _attention_case(rng, n_q, n_kv, d, dec_ctx, pre_len, pre_prefix, seed):
    b = sw.batch_from_lengths(dec_ctx, pre_len, pre_prefix, seed=seed, spare_blocks=3)
    shape = _shape(n_q, n_kv, d)
    T = b.n_tokens
    kp, vp = sw.make_kv_pool(shape, b.num_blocks, seed)
    # unused pool slots hold NaN canaries: masked keys must not leak them into outputs
    used = np.zeros((b.num_blocks, 16), bool)
    for r, n_keys in enumerate(b.cached_lens() + b.q_lens()):
        for p in range(int(n_keys)):
            used[b.block_table[r, p // 16], p % 16] = True
    kp.transpose(0, 3, 1, 2, 4)[~used] = CANARY
    vp.transpose(0, 3, 1, 2)[~used] = CANARY
    qkv = rand_bf16(rng, (T, shape.qkv_rows), 1.3)
    return b, shape, qkv, kp, vp


@pytest.mark.parametrize("n_q,n_kv,d", [(4, 2, 64), (32, 8, 128), (8, 1, 128), (16, 1, 64)])
@pytest.mark.parametrize("split", [0, 1, 3, 64, 200])
def test_decode_attention(ctx, n_q, n_kv, d, split):
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool

    rng = np.random.default_rng(n_q * 100 + d + split)
    dec = np.concatenate([[0, 1, 15, 16, 17, 1023, 2047], rng.integers(0, 2500, 40)])
    b, shape, qkv, kp, vp = _attention_case(rng, n_q, n_kv, d, dec, [], [], seed=split + 1)
    T = b.n_tokens
    q = f64(qkv[:, : n_q * d]).reshape(T, n_q, d)
    ref = ol.attention_all(shape, b, q, kp, vp).reshape(T, n_q * d)
    out = torch.full((T, n_q * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    pool = DevicePool.from_host(kp, vp, "cuda")
    dqkv = _dev(qkv)
    log_case(f"decode attention n_q={n_q} n_kv={n_kv} d={d} split={split}")
    abi.nf_op_decode_attn(ctx, abi.make_cfg(shape), dqkv.data_ptr(), abi.HostBatch.from_batch(b), pool.desc,
                          out.data_ptr(), split, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = f64(_host(out))
    assert np.isfinite(got).all()
    assert rel_inf(got, ref) <= TOL


@pytest.mark.parametrize("nb,ring,grid", [(0, 0, 0), (1, 2, 0), (1, 3, 0), (1, 4, 0), (2, 2, 0), (2, 3, 0), (1, 2, 64),
                                          (2, 2, 37), (0, 0, 37)])
@pytest.mark.parametrize("n_q,n_kv,d", [(32, 8, 128), (16, 1, 64)])
def test_decode_attention_launch_configs(ctx, n_q, n_kv, d, nb, ring, grid):
    """Every supported (blocks per softmax step, ring depth) pair and bounded persistent
    grids give the oracle's result, for chunks shorter and longer than 64 blocks."""
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool

    rng = np.random.default_rng(nb * 10 + ring + grid)
    dec = np.concatenate([[0, 15, 16, 17, 1023, 1024, 2047, 2600], rng.integers(0, 2700, 30)])
    b, shape, qkv, kp, vp = _attention_case(rng, n_q, n_kv, d, dec, [], [], seed=nb + ring)
    T = b.n_tokens
    q = f64(qkv[:, : n_q * d]).reshape(T, n_q, d)
    ref = ol.attention_all(shape, b, q, kp, vp).reshape(T, n_q * d)
    pool = DevicePool.from_host(kp, vp, "cuda")
    dqkv = _dev(qkv)
    try:
        abi.nf_ctx_set_decode_launch(ctx, grid, nb, ring)
        for split in (0, 48, 300):
            out = torch.full((T, n_q * d), float("nan"), dtype=torch.bfloat16, device="cuda")
            log_case(f"decode attention nb={nb} ring={ring} grid={grid} split={split} n_q={n_q} d={d}")
            abi.nf_op_decode_attn(ctx, abi.make_cfg(shape), dqkv.data_ptr(), abi.HostBatch.from_batch(b), pool.desc,
                                  out.data_ptr(), split, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            got = f64(_host(out))
            assert np.isfinite(got).all()
            assert rel_inf(got, ref) <= TOL, (split, rel_inf(got, ref))
        # q = 0: every key gets weight exactly 1, so the output is the plain mean of the
        # request's values up to bf16 output rounding and fp32 summation; a key block
        # counted twice or skipped shifts that mean far more than the bound
        qkv0 = qkv.copy()
        qkv0[:, : n_q * d] = 0
        ref0 = ol.attention_all(shape, b, np.zeros((T, n_q, d)), kp, vp).reshape(T, n_q * d)
        vmax = np.abs(f64(vp[np.isfinite(f64(vp))])).max()
        dq0 = _dev(qkv0)
        for split in (0, 48, 300):
            out = torch.full((T, n_q * d), float("nan"), dtype=torch.bfloat16, device="cuda")
            log_case(f"uniform decode attention nb={nb} ring={ring} grid={grid} split={split} n_q={n_q} d={d}")
            abi.nf_op_decode_attn(ctx, abi.make_cfg(shape), dq0.data_ptr(), abi.HostBatch.from_batch(b), pool.desc,
                                  out.data_ptr(), split, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            got = f64(_host(out))
            bound = 2.0**-8 * np.abs(ref0) + 4e-4 * vmax
            bad = np.abs(got - ref0) > bound
            assert not bad.any(), (split, int(bad.sum()), np.argwhere(bad)[:4].tolist())
    finally:
        abi.nf_ctx_set_decode_launch(ctx, 0)


def test_decode_launch_rejects_unsupported_configs(ctx):
    from nano_intra_overlap_amd import abi

    for nb, ring in ((1, 1), (1, 5), (2, 4), (3, 2), (4, 2), (0, 2), (1, 0)):
        with pytest.raises(abi.NanoflowError):
            abi.nf_ctx_set_decode_launch(ctx, 0, nb, ring)


# prefill chunk lengths and cached prefixes: ragged tiles, a prefix that is not block
# aligned, and the lengths the 8B workload's draw reaches (445, 952 and its cap of 1024)
PREFILL_CASES = {
    "ragged": ([1, 15, 16, 17, 100, 300], [0, 0, 7, 0, 33, 0]),
    "cap1024": ([1024], [0]),
    "long_prefix": ([952, 445, 63], [0, 37, 200]),
}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
@pytest.mark.parametrize("n_q,n_kv,d", [(4, 2, 64), (32, 8, 128), (8, 1, 128)])
def test_prefill_attention(ctx, n_q, n_kv, d, case):
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool

    rng = np.random.default_rng(7 * n_q + d + len(case))
    pre_len, pre_prefix = PREFILL_CASES[case]
    b, shape, qkv, kp, vp = _attention_case(rng, n_q, n_kv, d, [5, 9], pre_len, pre_prefix, seed=11)
    T = b.n_tokens
    q = f64(qkv[:, : n_q * d]).reshape(T, n_q, d)
    ref = ol.attention_all(shape, b, q, kp, vp).reshape(T, n_q * d)
    out = torch.full((T, n_q * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    pool = DevicePool.from_host(kp, vp, "cuda")
    dqkv = _dev(qkv)
    log_case(f"prefill attention n_q={n_q} n_kv={n_kv} d={d} case={case}")
    abi.nf_op_prefill_attn(ctx, abi.make_cfg(shape), dqkv.data_ptr(), abi.HostBatch.from_batch(b), pool.desc,
                           out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = f64(_host(out))
    rows = np.arange(b.n_decode, T)
    assert np.isfinite(got[rows]).all()
    assert rel_inf(got[rows], ref[rows]) <= TOL
    # decode rows were not touched by the prefill op
    assert np.isnan(got[: b.n_decode]).all()
