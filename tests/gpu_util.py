"""Shared helpers of the GPU parity tests (inputs, comparisons)."""

from __future__ import annotations

import numpy as np

from oracle import layer as ol
from synth import workloads as sw

TOL = 1e-2  # max relative error, per output tensor: ||gpu - ref||_inf / ||ref||_inf


def rel_inf(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref))) / denom


def rel_rms(got, ref) -> float:
    """||gpu - ref||_2 / ||ref||_2 over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.sqrt(np.sum(ref * ref)))
    diff = float(np.sqrt(np.sum((got - ref) ** 2)))
    return diff / denom if denom else diff


def deep_tol(ref_bf16, ref_exact, measure=None) -> float:
    """Tolerance for a result that several layers feed: the larger of TOL and twice the
    distance between the oracle's bf16-storage and exact-storage results for the same
    inputs. Both are computed by the oracle alone. Any bf16-storage implementation differs
    from the exact result by rounding noise that the layers amplify; two such
    implementations may differ by the sum of their distances from it."""
    measure = measure or rel_inf
    return max(TOL, 2.0 * measure(ref_bf16, ref_exact))


def rand_bf16(rng, shape, scale=1.0) -> np.ndarray:
    return sw.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def f64(bits) -> np.ndarray:
    return ol.bf16_to_f64(bits)


def log_case(name: str):
    """Name the case on stdout before a GPU step (a fault then still identifies it)."""
    print(f"[gpu case] {name}", flush=True)


def oracle_subbatch(shape, b, w, x, sample, seed):
    """Run the oracle on the sampled requests with a compact pool of only their blocks
    (rows of different requests are independent, so a sub-batch reproduces their rows)."""
    sub = b.select(sample)
    ranges = ol.request_ranges(b)
    rows = np.concatenate([np.arange(ranges[r][0], ranges[r][1]) for r in sample])
    need = (sub.cached_lens() + sub.q_lens() + 15) // 16
    used = sorted({int(sub.block_table[i, j]) for i in range(sub.n_requests) for j in range(int(need[i]))})
    remap = {blk: i for i, blk in enumerate(used)}
    bt = np.full_like(sub.block_table, -1)
    for i in range(sub.n_requests):
        for j in range(int(need[i])):
            bt[i, j] = remap[int(sub.block_table[i, j])]
    compact = sw.Batch(sub.decode_ctx, sub.prefill_len, sub.prefill_prefix, bt, len(used))
    kp, vp = sw.make_kv_pool_blocks(shape, used, seed)
    ref = ol.layer_forward(shape, w, x[rows], compact, kp, vp)
    exact = ol.layer_forward(shape, w, x[rows], compact, kp, vp, storage="exact")
    ref["y_exact"] = exact["y"]
    return rows, used, compact, ref
