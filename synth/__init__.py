"""Seeded synthetic inputs for one decoder-layer iteration over a mixed dense batch.

This package generates inputs only: layer shapes, per-request lengths, block tables,
weights, hidden states and the contents of the paged KV pool before the iteration. It holds
none of the layer's arithmetic (no norm, projection, rotary, attention or FFN math, no slot
addressing), so that the CPU oracle and the GPU library can both consume it without sharing
any computation.
"""

from .workloads import (  # noqa: F401
    BLOCK_SIZE,
    Batch,
    Shape,
    Workload,
    WORKLOADS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_batch,
    make_kv_pool,
    make_kv_pool_blocks,
    make_weights,
    make_x,
    kv_std,
)
