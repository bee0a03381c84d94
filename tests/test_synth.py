"""The seeded input generators (no GPU): the counter-based generators give the same bits on
the host (numpy) and through torch, so a device-resident input and the oracle's host copy
of it agree without a device-to-host transfer."""

import numpy as np

from synth import workloads as sw


def test_kv_pool_host_and_torch_agree():
    shape = sw.WORKLOADS["tiny"].shape
    for layer in (0, 3):
        k, v = sw.make_kv_pool(shape, 9, 5, layer=layer)
        kt, vt = sw.make_kv_pool_torch(shape, 9, 5, layer=layer, chunk_blocks=4)
        assert np.array_equal(k, kt.numpy().view(np.uint16)) and np.array_equal(v, vt.numpy().view(np.uint16))
    k0, _ = sw.make_kv_pool(shape, 9, 5, layer=0)
    assert not np.array_equal(k0, sw.make_kv_pool(shape, 9, 5, layer=1)[0])


def test_counter_weights_host_and_torch_agree():
    shape = sw.WORKLOADS["tiny"].shape
    a = sw.make_weights_counter(shape, 3, 2)
    b = sw.make_weights_counter_torch(shape, 3, 2, chunk=1000)
    assert set(a) == set(b) == {"g_attn", "w_qkv", "w_o", "g_ffn", "w_gate_up", "w_down"}
    for name in a:
        assert np.array_equal(a[name], b[name].numpy().view(np.uint16)), name
    # an MoE shape: experts stacked, router rows with std 1/sqrt(H)
    moe = sw.WORKLOADS["tiny_moe"].shape
    am, bm = sw.make_weights_counter(moe, 3, 1), sw.make_weights_counter_torch(moe, 3, 1, chunk=5000)
    assert am["w_gate_up"].shape == (8, 2 * moe.ffn, moe.hidden) and am["w_down"].shape == (8, moe.hidden, moe.ffn)
    for name in am:
        assert np.array_equal(am[name], bm[name].numpy().view(np.uint16)), name
    r = sw.bf16_bits_to_f32(sw.make_weights_counter(sw.WORKLOADS["mixtral_8x7b_layer"].shape, 0, 0,
                                                    matrices=("w_router",))["w_router"]).astype(np.float64)
    assert abs(r.std() * np.sqrt(4096) - 1) < 0.02
    rows = sw.make_weights_counter(shape, 3, 2, rows={"w_o": [5, 7], "w_down": [0]}, matrices=("w_o", "w_down"))
    assert np.array_equal(rows["w_o"], a["w_o"][[5, 7]]) and np.array_equal(rows["w_down"], a["w_down"][[0]])
    assert set(rows) == {"w_o", "w_down"}


def test_counter_weights_statistics_and_independence():
    shape = sw.WORKLOADS["tiny"].shape
    w = sw.make_weights_counter(shape, 0, 0)
    assert np.array_equal(w["g_attn"], sw.f32_to_bf16_bits(np.ones(shape.hidden, np.float32)))
    f = sw.bf16_bits_to_f32(w["w_gate_up"]).astype(np.float64)
    assert abs(f.mean()) < 2e-4 and abs(f.std() / sw.WEIGHT_STD - 1) < 0.01
    assert np.abs(f).max() <= 3.47 * sw.WEIGHT_STD
    other = sw.bf16_bits_to_f32(sw.make_weights_counter(shape, 0, 1)["w_gate_up"]).astype(np.float64)
    assert abs(np.corrcoef(f.ravel(), other.ravel())[0, 1]) < 0.01  # layers draw independently
    q = sw.bf16_bits_to_f32(w["w_qkv"]).astype(np.float64).ravel()
    assert abs(np.corrcoef(q[:-1], q[1:])[0, 1]) < 0.02  # neighbouring entries independent


def test_counter_generator_past_2_pow_32_matches_between_host_and_torch():
    """Pools of more than 2^32 elements (the long-context workload) keep one value per
    element, the same through numpy and torch; below 2^32 nothing changes."""
    import torch

    k1, k2 = sw._keys(3, 1, 0)
    scale = float(sw._kv_scale(sw.WORKLOADS["llama3_8b_layer"].shape))
    idx = np.concatenate([np.arange(0, 64), np.arange(2**32 - 64, 2**32 + 64), np.arange(2**33 + 5, 2**33 + 69)])
    host = sw._kv_f32_from_counter(idx.astype(np.uint64), np.uint64(k1), np.uint64(k2), np.float32(scale), np,
                                   lambda s: s.astype(np.int64).astype(np.float32))
    dev = sw._kv_f32_from_counter(torch.from_numpy(idx.astype(np.int64)), k1, k2,
                                  torch.tensor(scale, dtype=torch.float32), torch, lambda s: s.to(torch.float32))
    assert np.array_equal(host, dev.numpy())
    # elements 2^32 apart differ (the high word reaches the hash)
    lo = host[:64]
    wrapped = sw._kv_f32_from_counter((idx[:64] + 2**32).astype(np.uint64), np.uint64(k1), np.uint64(k2),
                                      np.float32(scale), np, lambda s: s.astype(np.int64).astype(np.float32))
    assert (lo != wrapped).mean() > 0.9
