"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a value printed on the pages, a
library routine, an invariant of the mathematics, or a brute-force computation built a
different way, chosen so that a plausible slip (dropped term, wrong sign or index,
transposed operand, wrong head grouping, wrong slot) fails at least one of them.
"""

import json
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest
import scipy.special
import torch

from oracle import layer as ol
from synth import workloads as sw

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def _cfg(**kw):
    base = dict(hidden=32, n_q=4, n_kv=2, head_dim=16, ffn=48, block_size=16, rms_eps=1e-5,
                rope_base=10000.0)
    base.update(kw)
    return SimpleNamespace(**base)


def _bf16_exact(rng, shape, scale=1.0):
    """float64 values that are exactly representable in bf16."""
    return ol.bf16_to_f64(sw.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale))


# ----------------------------------------------------------------------------- bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    vals = (rng.standard_normal(200000) * 10).astype(np.float32)
    # exact ties between two bf16 neighbours (low 16 bits = 0x8000) with both parities
    ties = (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    vals = np.concatenate([vals, ties.view(np.float32), np.float32([0.0, -0.0, 1e-30, -3e30])])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = ol.f64_to_bf16(vals.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(ol.bf16_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# ----------------------------------------------------------------------------- FLOPs


def test_flop_counter_reproduces_table2_ug():
    g = GOLDEN["table2_ug_gflop"]
    cfg = _cfg(hidden=g["shape"]["hidden"], ffn=g["shape"]["ffn"], n_q=64, n_kv=8, head_dim=128)
    ug = ol.op_flops(cfg, g["shape"]["dense_batch"])["ug"] * g["shape"]["n_layers"]
    assert ug == 153_931_627_888_640
    assert round(ug / 1e9, 1) == g["value"]


def test_layer_flops_equals_two_params_per_token_plus_attention():
    # closed form: 2 T P_layer + sum over (query head, visible key) of 4 d
    cfg = _cfg()
    b = sw.batch_from_lengths([5, 0, 17], [4, 9], [0, 3], seed=1)
    P = cfg.hidden * (cfg.n_q + 2 * cfg.n_kv) * cfg.head_dim + cfg.n_q * cfg.head_dim * cfg.hidden \
        + 3 * cfg.hidden * cfg.ffn
    T = b.n_tokens
    att = 4 * cfg.head_dim * cfg.n_q * ((5 + 1) + (0 + 1) + (17 + 1) + 4 * 5 // 2 + (4 + 5 + 6 + 7 + 8 + 9 + 10 + 11 + 12))
    assert ol.layer_flops(cfg, b) == 2 * T * P + att


# ----------------------------------------------------------------------------- norm / rope / swiglu / linear


def test_rmsnorm_constant_row_closed_form():
    c = 3.25
    g = np.linspace(0.5, 2.0, 64)
    out = ol.rmsnorm(np.full((1, 64), c), g, 1e-5)
    assert np.allclose(out[0], g * c / math.sqrt(c * c + 1e-5), rtol=1e-15, atol=0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 128))
    a = ol.rmsnorm(x, np.ones(128), 0.0)
    b = ol.rmsnorm(13.0 * x, np.ones(128), 0.0)
    assert np.allclose(a, b, rtol=1e-13)
    assert np.allclose(np.sqrt(np.mean(a * a, axis=1)), 1.0, rtol=1e-13)


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 2, 16))
    assert np.array_equal(ol.rope(x, np.zeros(3, np.int64), 10000.0), x)


def test_rope_matches_complex_rotation():
    # rotate-half pairs (i, i + d/2) rotate like complex numbers x_i + j x_{i+d/2} by pos*theta_i
    rng = np.random.default_rng(4)
    d = 16
    x = rng.standard_normal((5, 3, d))
    pos = np.array([0, 1, 7, 100, 4095])
    out = ol.rope(x, pos, 10000.0)
    z = x[..., : d // 2] + 1j * x[..., d // 2 :]
    theta = pos[:, None] * np.power(10000.0, -np.arange(0, d, 2) / d)[None, :]
    zr = z * np.exp(1j * theta)[:, None, :]
    assert np.allclose(out[..., : d // 2], zr.real, atol=1e-12)
    assert np.allclose(out[..., d // 2 :], zr.imag, atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))
    dots = []
    for m, n in [(10, 3), (107, 100), (2007, 2000)]:
        dots.append(float(np.sum(ol.rope(q, [m], 10000.0) * ol.rope(k, [n], 10000.0))))
    assert np.allclose(dots, dots[0], rtol=1e-9)
    norm = np.linalg.norm(ol.rope(q, [123], 10000.0)[0, 0].reshape(2, 16), axis=0)
    assert np.allclose(norm, np.linalg.norm(q[0, 0].reshape(2, 16), axis=0))


def test_silu_and_swiglu():
    z = np.linspace(-30, 30, 601)
    assert np.allclose(ol.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert ol.silu(np.array([0.0]))[0] == 0.0
    assert abs(ol.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(ol.silu(np.array([-40.0]))[0]) < 1e-15
    gate = np.array([[1.0, -2.0, 0.0]])
    up = np.array([[3.0, 5.0, 7.0]])
    got = ol.swiglu(np.concatenate([gate, up], axis=1), 3)
    assert np.allclose(got, scipy.special.expit(gate) * gate * up)


def test_linear_uses_out_in_layout():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 9))
    perm = np.array([8, 0, 3, 3, 5])  # output j picks input perm[j]
    w = np.zeros((5, 9))
    w[np.arange(5), perm] = 1.0
    assert np.array_equal(ol.linear(x, w), x[:, perm])


# ----------------------------------------------------------------------------- slots


def test_new_token_slots_match_block_expansion():
    b = sw.batch_from_lengths([0, 15, 16, 33], [17, 40], [0, 5], seed=7)
    # expand each request's table into a per-position list of (block, offset) pairs
    expected = []
    for r, (cached, qlen) in enumerate(zip(b.cached_lens(), b.q_lens())):
        per_pos = [(int(blk), off) for blk in b.block_table[r] if blk >= 0 for off in range(16)]
        expected += per_pos[cached : cached + qlen]
    assert ol.new_token_slots(b, 16) == expected


def test_write_kv_touches_exactly_the_new_slots():
    cfg = _cfg()
    b = sw.batch_from_lengths([3, 20, 31], [19], [2], seed=8)
    canary = np.uint16(0x7FC1)  # a NaN pattern that rounding of finite values never yields
    kp = ol.k_pool_from_tokens(np.full((b.num_blocks, cfg.n_kv, 16, cfg.head_dim), canary, np.uint16))
    vp = np.full((b.num_blocks, cfg.n_kv, cfg.head_dim, 16), canary, np.uint16)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((b.n_tokens, cfg.n_kv, cfg.head_dim))
    v = rng.standard_normal((b.n_tokens, cfg.n_kv, cfg.head_dim))
    k2, v2 = ol.write_kv(kp, vp, b, 16, k, v)
    changed_k = {(int(i), int(o)) for i, _, _, o, _ in zip(*np.nonzero(k2 != canary))}
    changed_v = {(int(i), int(o)) for i, _, _, o in zip(*np.nonzero(v2 != canary))}
    want = set(ol.new_token_slots(b, 16))
    assert changed_k == want and changed_v == want
    # every written entry of each token holds that token's rounded vector
    for t, (blk, off) in enumerate(ol.new_token_slots(b, 16)):
        assert np.array_equal(ol.k_tokens(k2)[blk, :, off, :], ol.f64_to_bf16(k[t]))
        assert np.array_equal(v2[blk, :, :, off], ol.f64_to_bf16(v[t]))


def test_key_pool_layout_is_column_chunks_of_32():
    # written by hand: dim i of token `off` of KV head g in block blk sits at [blk, g, i // 32, off, i % 32]
    b = sw.batch_from_lengths([5], [], seed=1, spare_blocks=0)
    d, n_kv = 64, 2
    kp = np.zeros((b.num_blocks, n_kv, 2, 16, 32), np.uint16)
    vp = np.zeros((b.num_blocks, n_kv, d, 16), np.uint16)
    k = np.arange(n_kv * d, dtype=np.float64).reshape(1, n_kv, d)
    k2, _ = ol.write_kv(kp, vp, b, 16, k, np.zeros_like(k))
    blk, off = ol.new_token_slots(b, 16)[0]
    assert off == 5
    for g in range(n_kv):
        for i in (0, 31, 32, 35, 63):
            assert ol.bf16_to_f64(k2[blk, g, i // 32, off, i % 32]) == g * d + i


def test_slot_rejects_bad_tables():
    b = sw.batch_from_lengths([20], [], seed=0)
    bad = sw.Batch(b.decode_ctx, b.prefill_len, b.prefill_prefix, b.block_table.copy(), b.num_blocks)
    bad.block_table[0, 1] = b.num_blocks
    with pytest.raises(IndexError):
        ol.new_token_slots(bad, 16)
    short = sw.Batch(b.decode_ctx, b.prefill_len, b.prefill_prefix, b.block_table[:, :1].copy(), b.num_blocks)
    with pytest.raises(IndexError):
        ol.new_token_slots(short, 16)


# ----------------------------------------------------------------------------- attention


def _paged_pool_from_sequences(b, seqs_k, seqs_v, n_kv, d):
    """Place each request's contiguous K/V sequence into its blocks, block by block."""
    kp = np.zeros((b.num_blocks, n_kv, 16, d), np.uint16)  # token-major, converted at the end
    vp = np.zeros((b.num_blocks, n_kv, d, 16), np.uint16)
    for r, (sk, sv) in enumerate(zip(seqs_k, seqs_v)):
        n = sk.shape[0]
        nblk = (n + 15) // 16
        pad = nblk * 16 - n
        sk = np.concatenate([sk, np.zeros((pad,) + sk.shape[1:])])
        sv = np.concatenate([sv, np.zeros((pad,) + sv.shape[1:])])
        for lb in range(nblk):
            blk = b.block_table[r, lb]
            kp[blk] = ol.f64_to_bf16(sk[lb * 16 : (lb + 1) * 16].transpose(1, 0, 2))
            vp[blk] = ol.f64_to_bf16(sv[lb * 16 : (lb + 1) * 16].transpose(1, 2, 0))
    return ol.k_pool_from_tokens(kp), vp


@pytest.mark.parametrize("n_q,n_kv", [(4, 2), (4, 1), (2, 2), (3, 3)])
def test_attention_matches_brute_force(n_q, n_kv):
    rng = np.random.default_rng(10 + n_q * 7 + n_kv)
    d = 16
    cfg = _cfg(n_q=n_q, n_kv=n_kv, head_dim=d)
    dec = [0, 1, 15, 16, 23]
    pre, pre_prefix = [1, 7, 17], [0, 0, 20]
    b = sw.batch_from_lengths(dec, pre, pre_prefix, seed=11)
    totals = list(b.cached_lens() + b.q_lens())
    seqs_k = [_bf16_exact(rng, (n, n_kv, d)) for n in totals]
    seqs_v = [_bf16_exact(rng, (n, n_kv, d)) for n in totals]
    kp, vp = _paged_pool_from_sequences(b, seqs_k, seqs_v, n_kv, d)
    q = rng.standard_normal((b.n_tokens, n_q, d))
    got = ol.attention_all(cfg, b, q, kp, vp)

    # brute force: whole score matrix of the dense batch over the concatenated sequences,
    # masked to same-request keys at or before the query position, softmax from scipy
    owner_k = np.concatenate([np.full(n, r) for r, n in enumerate(totals)])
    pos_k = np.concatenate([np.arange(n) for n in totals])
    K = np.concatenate(seqs_k)
    V = np.concatenate(seqs_v)
    owner_q = np.concatenate([np.full(int(ql), r) for r, ql in enumerate(b.q_lens())])
    pos_q = np.concatenate([np.arange(int(c), int(c) + int(ql)) for c, ql in zip(b.cached_lens(), b.q_lens())])
    mask = (owner_q[:, None] == owner_k[None, :]) & (pos_k[None, :] <= pos_q[:, None])
    want = np.zeros_like(got)
    for h in range(n_q):
        g = (h * n_kv) // n_q
        s = np.einsum("td,kd->tk", q[:, h], K[:, g]) / math.sqrt(d)
        s = np.where(mask, s, -np.inf)
        want[:, h] = scipy.special.softmax(s, axis=1) @ V[:, g]
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)


def test_attention_special_cases():
    d = 8
    rng = np.random.default_rng(12)
    # one key: output equals the value
    v = rng.standard_normal((1, 1, d))
    o = ol.attend(rng.standard_normal((1, 2, d)), rng.standard_normal((1, 1, d)), v, [0], 2, 1)
    assert np.allclose(o[0, 0], v[0, 0]) and np.allclose(o[0, 1], v[0, 0])
    # identical keys: uniform weights, output equals the mean of visible values
    keys = np.repeat(rng.standard_normal((1, 1, d)), 9, axis=0)
    vals = rng.standard_normal((9, 1, d))
    o = ol.attend(rng.standard_normal((2, 1, d)), keys, vals, [4, 8], 1, 1)
    assert np.allclose(o[0, 0], vals[:5, 0].mean(axis=0)) and np.allclose(o[1, 0], vals[:, 0].mean(axis=0))
    # GQA with replicated KV heads equals MHA
    q = rng.standard_normal((3, 4, d))
    k2 = rng.standard_normal((6, 2, d))
    v2 = rng.standard_normal((6, 2, d))
    gqa = ol.attend(q, k2, v2, [3, 4, 5], 4, 2)
    mha = ol.attend(q, np.repeat(k2, 2, axis=1), np.repeat(v2, 2, axis=1), [3, 4, 5], 4, 4)
    assert np.allclose(gqa, mha, rtol=1e-14)


# ----------------------------------------------------------------------------- whole layer


def _tiny_inputs(seed=0, gain_jitter=0.1):
    wl = sw.WORKLOADS["tiny"]
    b = sw.make_batch("tiny", seed)
    w = sw.make_weights(wl.shape, seed, gain_jitter=gain_jitter)
    x = sw.make_x(wl.shape, b.n_tokens, seed)
    kp, vp = sw.make_kv_pool(wl.shape, b.num_blocks, seed)
    return wl.shape, b, w, x, kp, vp


def test_layer_paged_equals_contiguous():
    shape, b, w, x, kp, vp = _tiny_inputs(1)
    ident = sw.make_batch("tiny", 1, shuffle=False)
    assert np.array_equal(ident.decode_ctx, b.decode_ctx)
    kp2 = np.zeros_like(kp)
    vp2 = np.zeros_like(vp)
    for r in range(b.n_requests):
        for lb in range(b.max_blocks):
            if b.block_table[r, lb] >= 0:
                kp2[ident.block_table[r, lb]] = kp[b.block_table[r, lb]]
                vp2[ident.block_table[r, lb]] = vp[b.block_table[r, lb]]
    for storage in ("exact", "bf16"):
        a = ol.layer_forward(shape, w, x, b, kp, vp, storage=storage)
        c = ol.layer_forward(shape, w, x, ident, kp2, vp2, storage=storage)
        assert np.array_equal(a["y"], c["y"])
    for r in range(b.n_requests):
        for lb in range(b.max_blocks):
            if b.block_table[r, lb] >= 0:
                assert np.array_equal(a["k_pool"][b.block_table[r, lb]], c["k_pool"][ident.block_table[r, lb]])
                assert np.array_equal(a["v_pool"][b.block_table[r, lb]], c["v_pool"][ident.block_table[r, lb]])


@pytest.mark.parametrize("storage", ["exact", "bf16"])
def test_layer_request_subset_invariance(storage):
    shape, b, w, x, kp, vp = _tiny_inputs(2)
    full = ol.layer_forward(shape, w, x, b, kp, vp, storage=storage)
    ranges = ol.request_ranges(b)
    for subset in ([0, 5, 14], [3, 15], [1, 2, 4, 6, 8, 10, 12]):
        sub = b.select(subset)
        rows = np.concatenate([np.arange(ranges[r][0], ranges[r][1]) for r in sorted(subset)])
        part = ol.layer_forward(shape, w, x[rows], sub, kp, vp, storage=storage)
        # bf16 storage: a last-bit difference of the matmul may flip one rounding (2^-8 relative)
        tol = 1e-12 if storage == "exact" else 2.0**-7
        assert np.allclose(part["y"], full["y"][rows], rtol=tol, atol=1e-12)
        assert np.allclose(part["attn"], full["attn"][rows], rtol=tol, atol=1e-12)


def test_layer_decode_equals_last_prefill_row():
    # prefilling L tokens == prefilling L-1 tokens, then decoding the last one at ctx L-1
    shape = sw.WORKLOADS["tiny"].shape
    L = 21
    w = sw.make_weights(shape, 3, gain_jitter=0.1)
    x = sw.make_x(shape, L, 3)
    one = sw.batch_from_lengths([], [L], seed=3, spare_blocks=0)
    kp = np.zeros((one.num_blocks, shape.n_kv, shape.head_dim // 32, 16, 32), np.uint16)
    vp = np.zeros((one.num_blocks, shape.n_kv, shape.head_dim, 16), np.uint16)
    full = ol.layer_forward(shape, w, x, one, kp, vp, storage="exact")
    first = sw.Batch(np.zeros(0, np.int32), np.array([L - 1], np.int32), np.zeros(1, np.int32),
                     one.block_table, one.num_blocks)
    part = ol.layer_forward(shape, w, x[: L - 1], first, kp, vp, storage="exact")
    dec = sw.Batch(np.array([L - 1], np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
                   one.block_table, one.num_blocks)
    last = ol.layer_forward(shape, w, x[L - 1 :], dec, part["k_pool"], part["v_pool"], storage="exact")
    assert np.allclose(last["y"][0], full["y"][L - 1], rtol=1e-12, atol=1e-12)
    assert np.array_equal(last["k_pool"], full["k_pool"])
    assert np.array_equal(last["v_pool"], full["v_pool"])


def test_layer_zero_projections_pass_residual_through():
    shape, b, w, x, kp, vp = _tiny_inputs(4)
    w0 = dict(w)
    w0["w_o"] = np.zeros_like(w["w_o"])
    w0["w_down"] = np.zeros_like(w["w_down"])
    for storage in ("exact", "bf16"):
        out = ol.layer_forward(shape, w0, x, b, kp, vp, storage=storage)
        assert np.array_equal(out["y"], ol.bf16_to_f64(x))
        w1 = dict(w)
        w1["w_down"] = np.zeros_like(w["w_down"])
        out1 = ol.layer_forward(shape, w1, x, b, kp, vp, storage=storage)
        assert np.array_equal(out1["y"], out1["x1"])


def test_layer_value_head_routes_to_attention_output():
    # With W_q = 0 every score is 0, so each query averages the visible values; with the V
    # rows of W_qkv selecting hidden features, attention output is a causal running mean.
    shape, b, w, x, kp, vp = _tiny_inputs(5, gain_jitter=0.0)
    H, d, nq, nkv = shape.hidden, shape.head_dim, shape.n_q, shape.n_kv
    wq = ol.bf16_to_f64(w["w_qkv"]).copy()
    wq[: nq * d] = 0.0
    wq[(nq + nkv) * d :] = 0.0
    for j in range(nkv * d):
        wq[(nq + nkv) * d + j, j] = 1.0
    w2 = dict(w)
    w2["w_qkv"] = ol.f64_to_bf16(wq)
    out = ol.layer_forward(shape, w2, x, b, kp, vp, storage="exact")
    hv = ol.bf16_to_f64(ol.f64_to_bf16(out["h"][:, : nkv * d])).reshape(-1, nkv, d)
    for r, (s, e, cached, qlen) in enumerate(ol.request_ranges(b)):
        keys, vals = ol.gather_kv(kp, vp, b, 16, r, cached)
        hist = vals  # cached values from the pool
        seq = np.concatenate([hist, hv[s:e]])  # this iteration's values, as stored
        for i in range(qlen):
            want = seq[: cached + i + 1].mean(axis=0)  # [n_kv, d]
            got = out["attn"][s + i].reshape(nq, d)
            for h in range(nq):
                assert np.allclose(got[h], want[h // (nq // nkv)], rtol=1e-12, atol=1e-12)


def test_bf16_storage_model_rounds_every_handoff():
    """storage='bf16' stores each handed-over tensor in bf16 and stays within the bf16
    error budget of the exact model (each rounding is at most 2^-9 relative)."""
    shape, b, w, x, kp, vp = _tiny_inputs(6)
    e = ol.layer_forward(shape, w, x, b, kp, vp, storage="exact")
    r = ol.layer_forward(shape, w, x, b, kp, vp, storage="bf16")
    for name in ("h", "q", "attn", "x1", "h2", "a", "y"):
        assert np.array_equal(ol.store_bf16(r[name]), r[name]), name
        assert not np.array_equal(e[name], r[name]), name
    rel = np.max(np.abs(r["y"] - e["y"])) / np.max(np.abs(e["y"]))
    assert 0 < rel < 2e-2


# ---- layer stack -----------------------------------------------------------------------


def _stack_inputs(n_layers, seed=7):
    wl = sw.WORKLOADS["tiny"]
    b = sw.make_batch("tiny", seed)
    ws = [sw.make_weights(wl.shape, seed, gain_jitter=0.1, layer=l) for l in range(n_layers)]
    x = sw.make_x(wl.shape, b.n_tokens, seed)
    pools = [sw.make_kv_pool(wl.shape, b.num_blocks, seed, layer=l) for l in range(n_layers)]
    return wl.shape, b, ws, x, [p[0] for p in pools], [p[1] for p in pools]


def _slot_major(k_tok):
    """[num_blocks, n_kv, BS, d] -> [num_blocks, BS, n_kv, d] (indexable by (block, offset))."""
    return k_tok.transpose(0, 2, 1, 3)


def _zero_branches(w):
    z = dict(w)
    z["w_o"] = np.zeros_like(w["w_o"])
    z["w_down"] = np.zeros_like(w["w_down"])
    return z


def test_stack_of_identity_layers_returns_its_input():
    """With the O and Down projections zero every layer is the identity on the hidden
    state; each layer still writes this iteration's K/V into its own pool only, and layers
    with equal weights write equal K/V."""
    shape, b, ws, x, kps, vps = _stack_inputs(3)
    zs = [_zero_branches(ws[0])] * 2 + [_zero_branches(ws[2])]
    for storage in ("exact", "bf16"):
        out = ol.stack_forward(shape, zs, x, b, kps, vps, storage=storage)
        for y in out["ys"]:
            assert np.array_equal(y, ol.bf16_to_f64(x))
    slots = ol.new_token_slots(b, 16)
    new = np.zeros((b.num_blocks, 16), bool)
    new[[s_[0] for s_ in slots], [s_[1] for s_ in slots]] = True
    for l in range(3):
        kt, kt0 = _slot_major(ol.k_tokens(out["k_pools"][l])), _slot_major(ol.k_tokens(kps[l]))
        vt, vt0 = out["v_pools"][l], vps[l]
        assert np.array_equal(kt[~new], kt0[~new])  # only the new slots of its own pool
        assert np.array_equal(vt.transpose(0, 3, 1, 2)[~new], vt0.transpose(0, 3, 1, 2)[~new])
        assert not np.array_equal(kt[new], kt0[new])
    # layers 0 and 1 share weights: same new K/V though their pools differ elsewhere
    k0, k1, k2 = (_slot_major(ol.k_tokens(out["k_pools"][l])) for l in range(3))
    assert np.array_equal(k0[new], k1[new]) and not np.array_equal(k0[~new], k1[~new])
    assert not np.array_equal(k0[new], k2[new])


def test_stack_applies_each_layer_with_its_own_weights_and_pool():
    """An identity layer placed first or last leaves exactly the other layer's result."""
    shape, b, ws, x, kps, vps = _stack_inputs(2, seed=8)
    z = _zero_branches(ws[0])
    one = ol.layer_forward(shape, ws[1], x, b, kps[1], vps[1])
    first = ol.stack_forward(shape, [z, ws[1]], x, b, kps, vps)
    assert np.array_equal(first["y"], one["y"])
    assert np.array_equal(first["k_pools"][1], one["k_pool"]) and np.array_equal(first["v_pools"][1], one["v_pool"])
    last = ol.stack_forward(shape, [ws[1], z], x, b, kps[::-1], vps[::-1])
    assert np.array_equal(last["y"], one["y"])
    assert np.array_equal(last["k_pools"][0], one["k_pool"])
    # a single-layer stack is the layer
    single = ol.stack_forward(shape, [ws[1]], x, b, [kps[1]], [vps[1]])
    assert np.array_equal(single["y"], one["y"])


def test_stack_flops_are_layers_times_layer_flops():
    shape, b, ws, x, kps, vps = _stack_inputs(3, seed=9)
    out = ol.stack_forward(shape, ws, x, b, kps, vps)
    H, F, d, nq, nkv = shape.hidden, shape.ffn, shape.head_dim, shape.n_q, shape.n_kv
    params = H * (nq + 2 * nkv) * d + nq * d * H + 3 * H * F
    attn = sum(4 * nq * d * (int(c) + 1) for c in b.decode_ctx) + sum(
        4 * nq * d * int(L) * (int(L) + 1) // 2 for L in b.prefill_len)
    assert out["flops"] == 3 * (2 * b.n_tokens * params + attn)


# ---- mixture-of-experts FFN --------------------------------------------------------------


def test_moe_route_matches_brute_force_and_breaks_ties_low():
    rng = np.random.default_rng(21)
    logits = rng.standard_normal((60, 8))
    logits[0] = [0.5, 2.0, 2.0, -1, 0, 2.0, 0, 0]  # three-way tie: experts 1 and 2 win, in that order
    logits[1] = [1.0] * 8                           # all equal: experts 0 and 1, weights 1/2
    sel, w = ol.moe_route(logits, 2)
    for t in range(60):
        ranked = sorted(range(8), key=lambda e: (-logits[t, e], e))[:2]
        assert sel[t].tolist() == ranked
        l0, l1 = logits[t, ranked[0]], logits[t, ranked[1]]
        assert np.isclose(w[t, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)
        assert np.isclose(w[t].sum(), 1.0, rtol=1e-15)
    assert sel[0].tolist() == [1, 2] and np.allclose(w[0], 0.5)
    assert sel[1].tolist() == [0, 1] and np.allclose(w[1], 0.5)


def _moe_inputs(seed=0):
    wl = sw.WORKLOADS["tiny_moe"]
    b = sw.make_batch("tiny_moe", seed)
    w = sw.make_weights(wl.shape, seed, gain_jitter=0.1)
    x = sw.make_x(wl.shape, b.n_tokens, seed)
    kp, vp = sw.make_kv_pool(wl.shape, b.num_blocks, seed)
    return wl.shape, b, w, x, kp, vp


def test_moe_with_identical_experts_is_the_dense_ffn():
    """Every expert the same FFN: the routing weights sum to one, so the layer is the dense
    layer with that FFN."""
    import dataclasses

    shape, b, w, x, kp, vp = _moe_inputs(1)
    same = dict(w)
    same["w_gate_up"] = np.stack([w["w_gate_up"][3]] * shape.n_experts)
    same["w_down"] = np.stack([w["w_down"][3]] * shape.n_experts)
    dense_shape = dataclasses.replace(shape, n_experts=0, top_k=0)
    dense_w = {k: v for k, v in w.items() if k != "w_router"}
    dense_w["w_gate_up"], dense_w["w_down"] = w["w_gate_up"][3], w["w_down"][3]
    moe = ol.layer_forward(shape, same, x, b, kp, vp, storage="exact")
    dense = ol.layer_forward(dense_shape, dense_w, x, b, kp, vp, storage="exact")
    assert np.allclose(moe["y"], dense["y"], rtol=1e-12, atol=1e-12)


def test_moe_is_invariant_to_renumbering_experts():
    shape, b, w, x, kp, vp = _moe_inputs(2)
    perm = np.array([5, 2, 7, 0, 3, 6, 1, 4])
    wp = dict(w)
    for k in ("w_gate_up", "w_down", "w_router"):
        wp[k] = w[k][perm]
    for storage in ("exact", "bf16"):
        a = ol.layer_forward(shape, w, x, b, kp, vp, storage=storage)
        c = ol.layer_forward(shape, wp, x, b, kp, vp, storage=storage)
        assert np.array_equal(a["y"], c["y"])
        assert np.array_equal(perm[c["moe_sel"]], a["moe_sel"])


def test_moe_token_output_depends_only_on_its_chosen_experts():
    shape, b, w, x, kp, vp = _moe_inputs(3)
    base = ol.layer_forward(shape, w, x, b, kp, vp)
    e = 4
    w2 = dict(w)
    w2["w_down"] = w["w_down"].copy()
    w2["w_down"][e] = sw.make_weights(shape, 99)["w_down"][e]
    out = ol.layer_forward(shape, w2, x, b, kp, vp)
    routed = (base["moe_sel"] == e).any(axis=1)
    assert routed.any() and (~routed).any()
    assert np.array_equal(out["y"][~routed], base["y"][~routed])
    assert (out["y"][routed] != base["y"][routed]).any(axis=1).all()
    # doubling expert e's down projection (exact in bf16) adds, to each token routed to e,
    # its routing weight for e times that expert's output
    w3 = dict(w)
    w3["w_down"] = w["w_down"].copy()
    w3["w_down"][e] = sw.f32_to_bf16_bits(2.0 * sw.bf16_bits_to_f32(w["w_down"][e]))
    ex = ol.layer_forward(shape, w, x, b, kp, vp, storage="exact")
    ex3 = ol.layer_forward(shape, w3, x, b, kp, vp, storage="exact")
    tok, slot = np.nonzero(ex["moe_sel"] == e)
    gu, down = ol.bf16_to_f64(w["w_gate_up"][e]), ol.bf16_to_f64(w["w_down"][e])
    o = ol.linear(ol.swiglu(ol.linear(ex["h2"][tok], gu), shape.ffn), down)
    assert np.allclose(ex3["y"][tok] - ex["y"][tok], ex["moe_wts"][tok, slot][:, None] * o, rtol=1e-9, atol=1e-12)


def test_moe_flops_closed_form():
    shape, b, w, x, kp, vp = _moe_inputs(4)
    out = ol.layer_forward(shape, w, x, b, kp, vp)
    H, F, d, nq, nkv, E = shape.hidden, shape.ffn, shape.head_dim, shape.n_q, shape.n_kv, shape.n_experts
    T = b.n_tokens
    attn = sum(4 * nq * d * (int(c) + 1) for c in b.decode_ctx) + sum(
        4 * nq * d * int(L) * (int(L) + 1) // 2 for L in b.prefill_len)
    want = 2 * T * (H * (nq + 2 * nkv) * d + nq * d * H) + 2 * T * 2 * 3 * H * F + 2 * T * E * H + attn
    assert out["flops"] == want


# ---- KV offload / reload ------------------------------------------------------------------


def test_kv_offload_is_the_attention_history_of_the_request():
    """Offloading a request's positions 0..n-1 yields, in order, exactly the keys and values
    attention gathers for it."""
    from oracle import kvio

    shape, b, w, x, kp, vp = _tiny_inputs(7)
    for r in (0, 3, b.n_requests - 1):
        n = int(b.cached_lens()[r])
        rows = kvio.offload(kp, vp, [0], [n], b.block_table[r:r + 1])
        keys, vals = ol.gather_kv(kp, vp, b, 16, r, n)
        assert np.array_equal(ol.bf16_to_f64(rows[:, 0]), keys)
        assert np.array_equal(ol.bf16_to_f64(rows[:, 1]), vals)


def test_kv_reload_round_trip_into_other_blocks():
    """A request's KV offloaded from one set of pages and reloaded into another (as for a
    follow-up round) reads back identically; every other slot of the new pool is untouched."""
    from oracle import kvio

    shape = sw.WORKLOADS["tiny"].shape
    kp, vp = sw.make_kv_pool(shape, 12, 1)
    kq, vq = sw.make_kv_pool(shape, 12, 2)
    t_a = np.array([[3, 7, 1, 9]])
    t_b = np.array([[10, 0, 5, 2]])
    rows = kvio.offload(kp, vp, [5], [50], t_a)
    k2, v2 = kvio.reload(kq, vq, [5], [50], t_b, rows)
    assert np.array_equal(kvio.offload(k2, v2, [5], [50], t_b), rows)
    moved = set(kvio.range_slots([5], [50], t_b))
    kt2, ktq = ol.k_tokens(k2), ol.k_tokens(kq)
    for blk in range(12):
        for off in range(16):
            if (blk, off) not in moved:
                assert np.array_equal(kt2[blk, :, off], ktq[blk, :, off])
                assert np.array_equal(v2[blk, :, :, off], vq[blk, :, :, off])
    with pytest.raises(ValueError):
        kvio.reload(kq, vq, [0, 0], [4, 4], np.array([[1], [1]]), np.zeros((8, 2, 2, 64), np.uint16))


# ---- analytical cost model -----------------------------------------------------------

from oracle import costmodel as cm  # noqa: E402


def test_eq5_reproduces_the_pages_70b_example():
    g = GOLDEN["eq5_example"]
    v = cm.optimal_throughput(g["compute_flops"], g["params"])
    assert abs(v - g["approx_tokens_per_s"]) / g["approx_tokens_per_s"] < 0.01
    # the quoted 1857 corresponds to a profiled peak of about 260 TFLOP/s, below 280
    assert cm.optimal_throughput(260e12, g["params"]) == pytest.approx(g["quoted"], rel=0.001)


def test_kv_bytes_per_token_matches_the_pages():
    for g in GOLDEN["kv_bytes_per_token"]:
        assert cm.kv_bytes_per_token(g["n_layers"], g["n_kv"], g["head_dim"], g["dtype_bytes"]) == g["value"], g


def test_effective_decode_intensity_matches_the_roofline_lesson():
    for g in GOLDEN["effective_decode_intensity"]:
        v = cm.decode_effective_intensity(g["params"], g["batch"], g["live_tokens"], g["kv_bytes_per_token"],
                                          g["weight_bytes_per_param"])
        assert round(v) == g["approx"], (g, v)
    # with no KV the intensity is the batch size (the lesson's "decode intensity ~ B")
    assert cm.decode_effective_intensity(8e9, 64, 0, 131072) == pytest.approx(64.0)


def test_eq4_factored_form_equals_time_ratio():
    # Equation 4 is T_mem / T_compute rearranged; check on unrelated numbers
    compute, bw, size, params, b = 2.5e15, 8e12, 288e9, 8.03e9, 2048
    tr = cm.tr_ratio(compute, bw, size, params, b)
    assert tr == pytest.approx(cm.t_mem(size, bw) / cm.t_compute(b, params, compute), rel=1e-12)
    assert 2.6 < tr < 2.8  # an 8B model on one 288 GB / 8 TB/s / 2.5 PF device is memory-bound
    # more tokens per batch lowers TR proportionally
    assert cm.tr_ratio(compute, bw, size, params, 2 * b) == pytest.approx(tr / 2)


def test_net_to_compute_ratio_is_the_ratio_of_the_two_times():
    # "Compute" and "NetBW" are aggregates over the tensor-parallel group in both forms
    d, layers, n_gpu, s = 8192, 80, 8, 2
    params = 12 * d * d * layers  # the page's P ~ 12 D^2 L
    compute, net_bw, b = 8 * 312e12, 8 * 300e9, 2048
    r = cm.net_to_compute(d, layers, params, n_gpu, compute, net_bw, s)
    ratio = cm.t_net(n_gpu, b, d, s, layers, net_bw) / cm.t_compute(b, params, compute)
    assert ratio == pytest.approx(r, rel=1e-12)
    assert 2 * d * layers / params == pytest.approx(1 / (6 * d))
