"""The pages' analytical cost model, as plain arithmetic — TEST INFRASTRUCTURE ONLY.

Follows "NanoFlow: Towards Optimal Large Language Model Serving Throughput" (paper-graph-ui
summary page, "The Cost Model and the Compute-Bound Classification"): memory time, compute
time, network time, the classification ratio TR (Equation 4), the network-to-compute ratio
and the optimal throughput (Equation 5); and "LLM Inference Performance" (KV-cache sizing,
and the roofline of batched decode with the effective-intensity formula that charges each
sequence's own KV stream).

Units are SI throughout: bytes, FLOP, seconds, bytes/s, FLOP/s.

Parity pins (not-gpu tests): Equation 5 on the page's 70B example, the three KV-per-token
sizes the pages print, the two effective decode intensities the roofline lesson prints, and
Equation 4's approximate form against the ratio of the memory and compute times it is
derived from.
"""

from __future__ import annotations


def t_mem(mem_size_bytes: float, mem_bw: float) -> float:
    """Memory time of one iteration: the whole device memory (weights + KV) streamed once."""
    return mem_size_bytes / mem_bw


def t_compute(dense_batch: float, params: float, compute: float) -> float:
    """Compute time of the dense operations: two FLOPs per parameter per token of the batch."""
    return 2.0 * dense_batch * params / compute


def t_net(n_gpu: int, dense_batch: float, d_model: int, s_type: int, n_layers: int, net_bw: float) -> float:
    """Network time of tensor parallelism: about four activation volumes per layer per GPU."""
    return 4.0 * n_gpu * dense_batch * d_model * s_type * n_layers / net_bw


def tr_ratio(compute: float, mem_bw: float, mem_size_bytes: float, params: float, dense_batch: float) -> float:
    """Equation 4: TR = T_mem / T_compute in its factored form
    (Compute / MemBW) * (MemSize / P_model) * 1 / (2 B_dense). TR > 1: memory-bound."""
    return (compute / mem_bw) * (mem_size_bytes / params) / (2.0 * dense_batch)


def net_to_compute(d_model: int, n_layers: int, params: float, n_gpu: int, compute: float, net_bw: float,
                   s_type: int) -> float:
    """T_net / T_compute = (2 D_model L / P_model) * (N_GPU * Compute / (NetBW / S_type))."""
    return (2.0 * d_model * n_layers / params) * (n_gpu * compute / (net_bw / s_type))


def optimal_throughput(compute: float, params: float) -> float:
    """Equation 5: tokens/s at full compute utilisation, Compute / (2 P_model)."""
    return compute / (2.0 * params)


def kv_bytes_per_token(n_layers: int, n_kv: int, head_dim: int, dtype_bytes: int) -> int:
    """KV-cache bytes one token holds across all layers: K and V, every KV head."""
    return 2 * n_layers * n_kv * head_dim * dtype_bytes


def decode_effective_intensity(params: float, batch: int, live_tokens: int, kv_bytes: int,
                               weight_bytes_per_param: int = 2) -> float:
    """FLOP per byte of one batched decode step: B tokens x 2P FLOPs over the weights read
    once (P x weight bytes) plus every sequence's own KV (B x live tokens x KV bytes)."""
    flops = batch * 2.0 * params
    bytes_ = params * weight_bytes_per_param + batch * live_tokens * kv_bytes
    return flops / bytes_
