"""Oracle of KV-cache offload and reload between a paged pool and host memory (CPU).

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

What it follows: the summary page, "KV-cache management and offloading" — each token's K/V
is copied out to host memory, and for a follow-up round of a conversation the request's
K/V is loaded back into pool pages (which may be other pages than before). Only the data
movement is defined here; the page places of a token follow the paged-KV slot rule
(slot = table[r][pos // BS] * BS + pos % BS, "Inside nano-vLLM" / "LLM Inference
Performance").

Host layout (the library's boundary layout): the ranges in request order, per token K then
V, each [n_kv][d], bf16 bits. Pool layout as in oracle.layer (K in 32-dim column chunks,
V dim-major within a block).
"""

from __future__ import annotations

import numpy as np

from oracle import layer as ol


def range_slots(first, n_tokens, block_table, block_size: int = 16):
    """(block, offset) of every token of the ranges, in host-row order."""
    out = []
    for r, (p0, n) in enumerate(zip(first, n_tokens)):
        for p in range(int(p0), int(p0) + int(n)):
            out.append((int(block_table[r][p // block_size]), p % block_size))
    return out


def offload(k_pool, v_pool, first, n_tokens, block_table, block_size: int = 16):
    """Token-major host rows [n, 2, n_kv, d] (bf16 bits) of the ranges' K and V."""
    kt = ol.k_tokens(k_pool)  # [nb, n_kv, BS, d]
    slots = range_slots(first, n_tokens, block_table, block_size)
    n_kv, d = kt.shape[1], kt.shape[3]
    rows = np.zeros((len(slots), 2, n_kv, d), np.uint16)
    for i, (blk, off) in enumerate(slots):
        rows[i, 0] = kt[blk, :, off, :]
        rows[i, 1] = v_pool[blk, :, :, off]
    return rows


def reload(k_pool, v_pool, first, n_tokens, block_table, rows, block_size: int = 16):
    """Copies of the pools with the ranges' slots set from host rows [n, 2, n_kv, d]."""
    slots = range_slots(first, n_tokens, block_table, block_size)
    if len(set(slots)) != len(slots):
        raise ValueError("two tokens of the ranges share a slot")
    kt = ol.k_tokens(k_pool).copy()
    v_new = v_pool.copy()
    for i, (blk, off) in enumerate(slots):
        kt[blk, :, off, :] = rows[i, 0]
        v_new[blk, :, :, off] = rows[i, 1]
    return ol.k_pool_from_tokens(kt), v_new
