"""Oracle of one pre-norm decoder-layer iteration over a mixed dense batch (float64, CPU).

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

What it follows
---------------
* Layer op order — KQV projection, (rotary), attention, O projection, Up/Gate projection,
  Down projection — as listed in the NanoFlow summary page ("Operation classification":
  KQV generation, decode/prefill attention, O projection, Up/Gate/Down) and the slides'
  operation-classification slide of a decoder-only layer.
* Nano-batches are independent: every op except attention is row-wise, attention is
  per request (summary page, "The Intra-Device Parallelism Mechanism"). The oracle therefore
  computes the plain sequential layer; any nano-batch plan must reproduce it.
* Decode attention reads the request's cached K/V (summary page, memory-bound operations:
  decode attention loads the per-request KV-cache); prefill attention keeps request
  boundaries ("Inside nano-vLLM", prefill batching: attention must preserve request
  boundaries).
* Paged KV: fixed 16-token blocks, a per-request table from logical block to physical
  block ("LLM Inference Performance", PagedAttention: block table as page table); new K/V
  are written at slot = table[r][pos // BS] * BS + pos % BS ("Inside nano-vLLM": the slot
  mapping locates new KV stores).
* Dense-batch order: decode requests first, then prefill chunks (slides, batch formation).

Readings where the pages are silent (stated again in the design notes):
* RMSNorm before attention and before the FFN, eps from the layer shape (1e-5).
* Rotary embedding: rotate-half pairs (i, i + d/2), inv_freq_i = base^(-2i/d), angle =
  position * inv_freq, all d dims rotated; K is stored after rotation.
* Attention: scale 1/sqrt(d), causal within a request, no bias or window. A decode token at
  position ctx attends to keys 0..ctx, including its own. Keys and values are read from the
  pool after this iteration's writes, i.e. as stored (bfloat16).
* SwiGLU: silu(gate) * up with gate = the first F rows of the gate/up weight.
* bfloat16 rounding is round-to-nearest-even of the exact value.
* Numeric model "bf16 storage, fp32 accumulation": tensors passed between operations are
  stored in bfloat16; arithmetic inside an operation is exact here (float64, which bounds
  any fp32 accumulation). ``storage="exact"`` drops the between-op rounding.

Pool layout (the library's boundary layout): K [num_blocks, n_kv, d/32, BS, 32] (in a block,
the keys' dims in column chunks of 32, each chunk token-major; a head dim that is not a
multiple of 32 is a single chunk), V [num_blocks, n_kv, d, BS] (dim-major in a block). Both
hold bfloat16 bit patterns.

Parity pins: every function here is pinned by the not-gpu tests (brute-force attention on
tiny inputs, paged/contiguous invariance, request-subset invariance, decode/prefill
consistency, closed forms and special cases for norm, rotary, SwiGLU, projections and bf16
rounding, the FLOP count against the summary page's Table 2). The values of the whole
layer have no worked example on the pages: they rest on those pins.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------
# bfloat16 storage
# --------------------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint16, copy=False)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even) -> uint16 bit patterns.

    bfloat16 keeps 8 significant bits: with x = m * 2^e, m in [0.5, 1), neighbouring values
    are q = 2^(e - 8) apart, and never closer than the subnormal spacing 2^-133. x is
    rounded to the nearest multiple of q (rint rounds half to even; x / q is exact because
    q is a power of two), then re-expressed as float32, whose upper 16 bits are then
    exactly the bfloat16 pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x / q) * q
    f = r.astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------------------
# batch layout and paged-KV slots
# --------------------------------------------------------------------------------------


def request_ranges(batch):
    """Token range [start, end), cached length and new-token count of each request.

    Requests are the decodes (one new token each) followed by the prefill chunks.
    """
    n_dec = len(batch.decode_ctx)
    q_len = [1] * n_dec + [int(v) for v in batch.prefill_len]
    cached = [int(v) for v in batch.decode_ctx] + [int(v) for v in batch.prefill_prefix]
    out = []
    start = 0
    for r in range(len(q_len)):
        out.append((start, start + q_len[r], cached[r], q_len[r]))
        start += q_len[r]
    return out


def token_positions(batch):
    """Per token: owning request and position in that request's sequence."""
    req, pos = [], []
    for r, (start, end, cached, qlen) in enumerate(request_ranges(batch)):
        for i in range(qlen):
            req.append(r)
            pos.append(cached + i)
    return np.asarray(req, dtype=np.int64), np.asarray(pos, dtype=np.int64)


def slot(batch, block_size: int, r: int, pos: int):
    """(physical block, offset in block) of position ``pos`` of request ``r``."""
    lb = pos // block_size
    if lb >= batch.block_table.shape[1]:
        raise IndexError(f"request {r}: block table too short for position {pos}")
    blk = int(batch.block_table[r, lb])
    if blk < 0 or blk >= batch.num_blocks:
        raise IndexError(f"request {r}: block id {blk} out of range at position {pos}")
    return blk, pos % block_size


def new_token_slots(batch, block_size: int):
    """Slots written this iteration, one per token in dense-batch order."""
    req, pos = token_positions(batch)
    return [slot(batch, block_size, int(r), int(p)) for r, p in zip(req, pos)]


# --------------------------------------------------------------------------------------
# elementwise / row ops
# --------------------------------------------------------------------------------------


def rmsnorm(x, g, eps: float):
    """x / sqrt(mean(x^2) + eps) * g, per row."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def linear(x, w):
    """x @ w^T for a Linear-layout weight w [out, in]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def rope(x, pos, base: float):
    """Rotate-half rotary embedding of x [n, heads, d] at integer positions pos [n]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    theta = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(gu, ffn: int):
    """silu(gate) * up, where gate is the first ``ffn`` columns of gu and up the next."""
    return silu(gu[:, :ffn]) * gu[:, ffn:]


# --------------------------------------------------------------------------------------
# paged causal GQA attention
# --------------------------------------------------------------------------------------


def gather_kv(k_pool, v_pool, batch, block_size: int, r: int, n_keys: int):
    """Keys [n, n_kv, d] and values [n, n_kv, d] of positions 0..n-1 of request r (float64)."""
    p = np.arange(n_keys, dtype=np.int64)
    lb = p // block_size
    if n_keys and lb[-1] >= batch.block_table.shape[1]:
        raise IndexError(f"request {r}: block table too short for {n_keys} keys")
    blk = batch.block_table[r, lb].astype(np.int64)
    if np.any(blk < 0) or np.any(blk >= batch.num_blocks):
        raise IndexError(f"request {r}: block id out of range")
    off = p % block_size
    keys = k_pool[blk, :, :, off, :]  # advanced indices first: [n, n_kv, d/32, 32]
    keys = keys.reshape(keys.shape[0], keys.shape[1], keys.shape[2] * keys.shape[3])  # dim = chunk * c + j
    values = v_pool[blk, :, :, off]  # advanced indices first: [n, n_kv, d]
    return bf16_to_f64(keys), bf16_to_f64(values)


def attend(q, keys, values, q_pos, n_q: int, n_kv: int):
    """Causal softmax attention of queries q [m, n_q, d] at positions q_pos [m] over keys /
    values [n, n_kv, d] at positions 0..n-1; query head h uses KV head h // (n_q / n_kv)."""
    m, _, d = q.shape
    group = n_q // n_kv
    out = np.zeros((m, n_q, d))
    key_pos = np.arange(keys.shape[0])
    allowed = key_pos[None, :] <= np.asarray(q_pos)[:, None]
    for h in range(n_q):
        g = h // group
        s = (q[:, h, :] @ keys[:, g, :].T) / np.sqrt(d)
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ values[:, g, :]
    return out


# --------------------------------------------------------------------------------------
# KV write
# --------------------------------------------------------------------------------------


def write_kv(k_pool, v_pool, batch, block_size: int, k, v):
    """Copies of the pools with this iteration's K/V (float64 [T, n_kv, d]) stored as bf16."""
    k_new = k_pool.copy()
    v_new = v_pool.copy()
    kb = f64_to_bf16(k)
    vb = f64_to_bf16(v)
    for t, (blk, off) in enumerate(new_token_slots(batch, block_size)):
        k_new[blk, :, :, off, :] = kb[t].reshape(kb.shape[1], k_pool.shape[2], k_pool.shape[4])
        v_new[blk, :, :, off] = vb[t]
    return k_new, v_new


def k_tokens(k_pool):
    """Token-major view [num_blocks, n_kv, BS, d] of a key pool in the boundary layout."""
    nb, g, nc, bs, ch = k_pool.shape
    return k_pool.transpose(0, 1, 3, 2, 4).reshape(nb, g, bs, nc * ch)


def k_chunk(d: int) -> int:
    """Dims per key column chunk: 32 (the library's head dims are multiples of 32); a head dim
    that is not a multiple of 32 is one chunk (plain token-major)."""
    return 32 if d % 32 == 0 else d


def k_pool_from_tokens(k_tok):
    """Boundary layout [num_blocks, n_kv, d/c, BS, c] of token-major keys [.., BS, d]."""
    nb, g, bs, d = k_tok.shape
    c = k_chunk(d)
    return np.ascontiguousarray(k_tok.reshape(nb, g, bs, d // c, c).transpose(0, 1, 3, 2, 4))


# --------------------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------------------


def attention_all(cfg, batch, q, k_pool, v_pool):
    """Attention output [T, n_q, d] of every token, per request, over the stored pool."""
    T = q.shape[0]
    out = np.zeros((T, cfg.n_q, cfg.head_dim))
    for r, (start, end, cached, qlen) in enumerate(request_ranges(batch)):
        n_keys = cached + qlen
        keys, values = gather_kv(k_pool, v_pool, batch, cfg.block_size, r, n_keys)
        q_pos = cached + np.arange(qlen)
        out[start:end] = attend(q[start:end], keys, values, q_pos, cfg.n_q, cfg.n_kv)
    return out


def store_bf16(a):
    """A tensor stored between operations in bfloat16: round to nearest even, as float64."""
    return bf16_to_f64(f64_to_bf16(a))


def layer_forward(cfg, weights, x_bits, batch, k_pool, v_pool, storage: str = "bf16"):
    """One decoder-layer iteration.

    cfg     object with hidden, n_q, n_kv, head_dim, ffn, block_size, rms_eps, rope_base
    weights dict of bf16 bit arrays: g_attn [H], w_qkv [(n_q+2n_kv)d, H], w_o [H, n_q d],
            g_ffn [H], w_gate_up [2F, H], w_down [H, F]; for an MoE shape (cfg.n_experts = E
            > 0) w_gate_up [E, 2F, H], w_down [E, H, F], w_router [E, H] (see moe_ffn)
    x_bits  bf16 bits [T, H]
    batch   object with decode_ctx, prefill_len, prefill_prefix, block_table, num_blocks
    k_pool  bf16 bits [num_blocks, n_kv, d/32, BS, 32]; v_pool bf16 bits [num_blocks, n_kv, d, BS]
    storage "bf16": the numeric model of a bf16-storage layer — every tensor handed from one
            operation to the next (h, qkv, rotated q, attention output, x1, h2, a, y; K/V in
            the pool) is stored in bfloat16 (round to nearest even) and everything inside an
            operation is exact (float64). "exact": no rounding except the KV pool, which is
            bfloat16 storage by definition.

    Returns a dict: y (float64 [T, H]), k_pool / v_pool (updated copies), the intermediates
    h, q, k, v (after rotary), attn [T, n_q d], x1, h2, a (None for MoE), and flops (int);
    MoE layers add moe_sel, moe_wts, moe_logits (see moe_ffn).
    """
    return _layer(cfg, weights, bf16_to_f64(x_bits), batch, k_pool, v_pool, storage)


def _layer(cfg, weights, x, batch, k_pool, v_pool, storage):
    """layer_forward on a float64 input x [T, H]."""
    if storage not in ("bf16", "exact"):
        raise ValueError("storage must be 'bf16' or 'exact'")
    st = store_bf16 if storage == "bf16" else (lambda a: a)
    H, nq, nkv, d, F = cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn
    T = x.shape[0]
    W = {name: bf16_to_f64(val) for name, val in weights.items()}
    _, pos = token_positions(batch)
    if pos.shape[0] != T:
        raise ValueError(f"batch holds {pos.shape[0]} tokens but x has {T} rows")

    h = st(rmsnorm(x, W["g_attn"], cfg.rms_eps))
    qkv = st(linear(h, W["w_qkv"]))
    q = qkv[:, : nq * d].reshape(T, nq, d)
    k = qkv[:, nq * d : (nq + nkv) * d].reshape(T, nkv, d)
    v = qkv[:, (nq + nkv) * d :].reshape(T, nkv, d)
    q = st(rope(q, pos, cfg.rope_base))
    k = rope(k, pos, cfg.rope_base)
    k_new, v_new = write_kv(k_pool, v_pool, batch, cfg.block_size, k, v)
    attn = st(attention_all(cfg, batch, q, k_new, v_new).reshape(T, nq * d))
    x1 = st(x + linear(attn, W["w_o"]))
    h2 = st(rmsnorm(x1, W["g_ffn"], cfg.rms_eps))
    out = {}
    if getattr(cfg, "n_experts", 0):
        ffn, out["moe_sel"], out["moe_wts"], out["moe_logits"] = moe_ffn(h2, W, cfg, st)
        y = st(x1 + ffn)
        a = None
    else:
        a = st(swiglu(linear(h2, W["w_gate_up"]), F))
        y = st(x1 + linear(a, W["w_down"]))
    out.update({
        "y": y, "k_pool": k_new, "v_pool": v_new, "h": h, "q": q, "k": k, "v": v,
        "attn": attn, "x1": x1, "h2": h2, "a": a, "flops": layer_flops(cfg, batch),
    })
    return out


# --------------------------------------------------------------------------------------
# Mixture-of-experts FFN
# --------------------------------------------------------------------------------------


def moe_route(logits, top_k: int):
    """The top_k experts of every token by router logit, largest first (equal logits: the
    lower expert index first), and the softmax of the chosen logits.

    The summary page ("MoE models") adds a gate-routing operation in front of an FFN whose
    experts each compute on their own tokens; the routing rule itself (top-2 of the router
    logits, softmax over the chosen two) is the Mixtral-style reading of that operation.
    """
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    chosen = np.take_along_axis(logits, order, axis=1)
    w = np.exp(chosen - chosen[:, :1])
    return order, w / w.sum(axis=1, keepdims=True)


def moe_ffn(h2, W, cfg, st):
    """FFN of a mixture-of-experts layer on float64 h2 [T, H] with float64 weights W:
    w_router [E, H], w_gate_up [E, 2F, H], w_down [E, H, F]. Every expert is a SwiGLU FFN
    applied to the tokens routed to it (its rows of the grouped GEMM); the output of a token
    is the routing-weighted sum of its experts' outputs. ``st`` stores the tensors handed
    between operations (each expert's a and output) as for the dense FFN.

    Returns (ffn [T, H], chosen experts [T, top_k], weights [T, top_k], logits [T, E]).
    """
    F = cfg.ffn
    logits = linear(h2, W["w_router"])
    sel, wts = moe_route(logits, cfg.top_k)
    ffn = np.zeros_like(h2)
    for e in range(cfg.n_experts):
        tok, slot = np.nonzero(sel == e)
        if tok.size == 0:
            continue
        a = st(swiglu(linear(h2[tok], W["w_gate_up"][e]), F))
        o = st(linear(a, W["w_down"][e]))
        np.add.at(ffn, tok, wts[tok, slot][:, None] * o)
    return ffn, sel, wts, logits


def stack_forward(cfg, layer_weights, x_bits, batch, k_pools, v_pools, storage: str = "bf16"):
    """Several decoder layers end to end over one batch (one model iteration).

    The layers of a decoder-only model run in sequence, each on the previous one's output,
    and every layer keeps a KV cache of its own; the batch (positions, slots, block table)
    is the same for all of them (summary page, "The NanoFlow Runtime System": one iteration
    runs the whole model over the dense batch; slides "8B Pipeline Design": the next
    layer's KQV follows this layer's Down).

    layer_weights  list of weight dicts as for layer_forward, one per layer
    k_pools, v_pools  lists of per-layer pools (bf16 bits), as for layer_forward
    storage  as for layer_forward; with "bf16" the hidden state handed from one layer to the
             next is stored in bfloat16, with "exact" it is not rounded.

    Returns a dict: y (float64 [T, H]), k_pools / v_pools (updated copies, per layer),
    ys and attns (every layer's output and attention output), flops.
    """
    if not (len(layer_weights) == len(k_pools) == len(v_pools)) or not layer_weights:
        raise ValueError("one weight dict and one pool pair per layer, at least one layer")
    x = bf16_to_f64(x_bits)
    ys, attns, kps, vps, flops = [], [], [], [], 0
    for w, kp, vp in zip(layer_weights, k_pools, v_pools):
        out = _layer(cfg, w, x, batch, kp, vp, storage)
        x = out["y"]
        ys.append(x)
        attns.append(out["attn"])
        kps.append(out["k_pool"])
        vps.append(out["v_pool"])
        flops += out["flops"]
    return {"y": x, "ys": ys, "attns": attns, "k_pools": kps, "v_pools": vps, "flops": flops}


# --------------------------------------------------------------------------------------
# FLOP counter
# --------------------------------------------------------------------------------------


def matmul_flops(m: int, n: int, k: int) -> int:
    """2 m n k: one multiply and one add per weight element per row."""
    return 2 * int(m) * int(n) * int(k)


def op_flops(cfg, n_tokens: int) -> dict:
    """FLOPs of each projection of one layer at a dense batch of ``n_tokens`` rows (an MoE
    layer: the router, and Up/Gate/Down once per chosen expert of every token)."""
    H, nq, nkv, d, F = cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn
    E = getattr(cfg, "n_experts", 0)
    rows = n_tokens * (cfg.top_k if E else 1)
    out = {
        "kqv": matmul_flops(n_tokens, (nq + 2 * nkv) * d, H),
        "o": matmul_flops(n_tokens, H, nq * d),
        "ug": matmul_flops(rows, 2 * F, H),
        "down": matmul_flops(rows, H, F),
    }
    if E:
        out["router"] = matmul_flops(n_tokens, E, H)
    return out


def attention_flops(cfg, batch) -> int:
    """4 d per (query head, causally visible key): q.k and p.v, one multiply-add each."""
    total = 0
    for start, end, cached, qlen in request_ranges(batch):
        for i in range(qlen):
            total += 4 * cfg.head_dim * cfg.n_q * (cached + i + 1)
    return total


def layer_flops(cfg, batch) -> int:
    n_tokens = sum(e - s for s, e, _, _ in request_ranges(batch))
    return sum(op_flops(cfg, n_tokens).values()) + attention_flops(cfg, batch)
