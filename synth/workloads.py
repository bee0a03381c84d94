"""Workload definitions and seeded generators.

Every generator takes an integer seed and derives an independent numpy stream per input
kind (weights, hidden states, lengths, block permutation), so that changing one input's
recipe never shifts another's draws.

Values are produced as bfloat16 bit patterns held in ``uint16`` arrays, the storage type of
the layer's tensors. The KV pool history is produced by a counter-based hash so that any
block can be regenerated on its own (on the host with numpy, or on a device with torch
integer ops, bit-identically) without materialising the whole pool on the host.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
K_CHUNK = 32  # keys are stored in column chunks of this many dims (see make_kv_pool_blocks)


def _k_chunk(d: int) -> int:
    return K_CHUNK if d % K_CHUNK == 0 else d

# --------------------------------------------------------------------------------------
# bf16 storage helpers (input generation only)
# --------------------------------------------------------------------------------------


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) -> uint16 bits.

    Works chunk by chunk with one reused temporary so that large weight matrices do not
    allocate several full-size intermediates.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    flat = a.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, dtype=np.uint16)
    chunk = 1 << 22
    tmp = np.empty(min(chunk, flat.size), dtype=np.uint32)
    for i in range(0, flat.size, chunk):
        u = flat[i : i + chunk]
        t = tmp[: u.size]
        np.right_shift(u, 16, out=t)
        np.bitwise_and(t, 1, out=t)
        np.add(t, 0x7FFF, out=t)
        np.add(t, u, out=t)  # NaN payloads may wrap; they are patched below
        np.right_shift(t, 16, out=t)
        out[i : i + chunk] = t
        nan = np.isnan(u.view(np.float32))
        if nan.any():
            out[i : i + chunk][nan] = np.uint16(0x7FC0)
    return out.reshape(a.shape)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------------------
# shapes and workloads
# --------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Shape:
    """Shape of one pre-norm decoder layer with grouped-query attention and a SwiGLU FFN."""

    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    block_size: int = BLOCK_SIZE
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    n_layers: int = 1
    n_experts: int = 0  # 0 = dense FFN
    top_k: int = 0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim

    @property
    def q_width(self) -> int:
        return self.n_q * self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    n_tokens: int
    description: str
    # prefill chunks: "fixed" lengths, or a lognormal draw
    prefill_fixed: tuple = ()
    prefill_lognormal: tuple = ()  # (median, sigma, cap)
    n_decode_fixed: int | None = None  # else n_tokens - sum(prefill)
    decode_ctx_range: tuple = (0, 0)  # inclusive
    nano_sweep: tuple = (1, 2, 4)
    default_bounds: tuple | None = None  # nano-batch bounds used when no plan is given
    extra: dict = field(default_factory=dict)


TINY = Shape(hidden=256, n_q=4, n_kv=2, head_dim=64, ffn=688)
TINY_MOE = Shape(hidden=256, n_q=4, n_kv=2, head_dim=64, ffn=256, n_experts=8, top_k=2)
LLAMA3_8B = Shape(hidden=4096, n_q=32, n_kv=8, head_dim=128, ffn=14336)
LLAMA3_8B_X32 = Shape(hidden=4096, n_q=32, n_kv=8, head_dim=128, ffn=14336, n_layers=32)
LLAMA2_70B_TP8 = Shape(hidden=8192, n_q=8, n_kv=1, head_dim=128, ffn=3584)
MIXTRAL_8X7B = Shape(hidden=4096, n_q=32, n_kv=8, head_dim=128, ffn=14336, n_experts=8, top_k=2)

WORKLOADS = {
    "tiny": Workload(
        name="tiny",
        shape=TINY,
        n_tokens=78,
        description="tiny layer: 2 prefill x 32 + 14 decode, ctx U[16,128]",
        prefill_fixed=(32, 32),
        n_decode_fixed=14,
        decode_ctx_range=(16, 128),
        nano_sweep=(2,),
        default_bounds=(0, 39, 78),
    ),
    "tiny_moe": Workload(
        name="tiny_moe",
        shape=TINY_MOE,
        n_tokens=78,
        description="tiny MoE layer (8 experts, top 2): 2 prefill x 32 + 14 decode, ctx U[16,128]",
        prefill_fixed=(32, 32),
        n_decode_fixed=14,
        decode_ctx_range=(16, 128),
        nano_sweep=(2,),
        default_bounds=(0, 39, 78),
    ),
    "llama3_8b_layer": Workload(
        name="llama3_8b_layer",
        shape=LLAMA3_8B,
        n_tokens=2048,
        description="LLaMA-3-8B-shaped layer, 2048-token dense batch: 1 lognormal prefill "
        "chunk (median 512, cap 1024) + decode ctx U[256,2048]",
        prefill_lognormal=(512, 0.5, 1024),
        decode_ctx_range=(256, 2048),
        nano_sweep=(1, 2, 4),
    ),
    "llama3_8b_32layer": Workload(
        name="llama3_8b_32layer",
        shape=LLAMA3_8B_X32,
        n_tokens=2048,
        description="LLaMA-3-8B-shaped 32-layer stack, same dense-batch mix as the 8B layer",
        prefill_lognormal=(512, 0.5, 1024),
        decode_ctx_range=(256, 2048),
        nano_sweep=(1, 2, 4),
        extra={"layer_workload": "llama3_8b_layer"},
    ),
    "llama3_8b_longctx_layer": Workload(
        name="llama3_8b_longctx_layer",
        shape=LLAMA3_8B,
        n_tokens=2048,
        description="LLaMA-3-8B-shaped layer, 2048-token batch with long decode contexts: 1 lognormal "
        "prefill chunk (median 512, cap 1024) + decode ctx U[4096,16384] (attention-dominated)",
        prefill_lognormal=(512, 0.5, 1024),
        decode_ctx_range=(4096, 16384),
        nano_sweep=(1, 2, 4),
    ),
    "llama2_70b_tp8_layer": Workload(
        name="llama2_70b_tp8_layer",
        shape=LLAMA2_70B_TP8,
        n_tokens=2048,
        description="one GPU's TP-8 share of a LLaMA-2-70B layer: 1 prefill chunk of 512 + "
        "1536 decode, ctx U[512,4096]",
        prefill_fixed=(512,),
        decode_ctx_range=(512, 4096),
        nano_sweep=(1, 2, 4),
    ),
    "mixtral_8x7b_layer": Workload(
        name="mixtral_8x7b_layer",
        shape=MIXTRAL_8X7B,
        n_tokens=2048,
        description="Mixtral-8x7B-shaped MoE layer in the 8B-layer dense-batch mix",
        prefill_lognormal=(512, 0.5, 1024),
        decode_ctx_range=(256, 2048),
        nano_sweep=(1, 2, 4),
    ),
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


STREAM_WEIGHTS, STREAM_X, STREAM_LENGTHS, STREAM_BLOCKS = 1, 2, 3, 4

# --------------------------------------------------------------------------------------
# batch descriptor
# --------------------------------------------------------------------------------------


@dataclass
class Batch:
    """Per-request lengths and the block table of one dense batch.

    Requests are ordered decodes first, then prefill chunks. A decode request holds one new
    token and ``decode_ctx[i]`` tokens already cached; a prefill chunk holds
    ``prefill_len[j]`` new tokens after ``prefill_prefix[j]`` cached ones.
    ``block_table[r, i]`` is the physical block holding logical block ``i`` of request ``r``
    (-1 where unused).
    """

    decode_ctx: np.ndarray
    prefill_len: np.ndarray
    prefill_prefix: np.ndarray
    block_table: np.ndarray
    num_blocks: int

    @property
    def n_decode(self) -> int:
        return int(self.decode_ctx.shape[0])

    @property
    def n_prefill(self) -> int:
        return int(self.prefill_len.shape[0])

    @property
    def n_requests(self) -> int:
        return self.n_decode + self.n_prefill

    @property
    def n_tokens(self) -> int:
        return self.n_decode + int(self.prefill_len.sum())

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def q_lens(self) -> np.ndarray:
        return np.concatenate([np.ones(self.n_decode, np.int64), self.prefill_len.astype(np.int64)])

    def cached_lens(self) -> np.ndarray:
        return np.concatenate([self.decode_ctx.astype(np.int64), self.prefill_prefix.astype(np.int64)])

    def select(self, requests) -> "Batch":
        """Sub-batch of the given request indices (kept in the decode-then-prefill order).

        Block ids are kept, so the sub-batch reads the same pool as the full batch.
        """
        req = np.asarray(sorted(int(r) for r in requests), dtype=np.int64)
        dec = req[req < self.n_decode]
        pre = req[req >= self.n_decode] - self.n_decode
        rows = np.concatenate([dec, pre + self.n_decode])
        return Batch(
            decode_ctx=self.decode_ctx[dec].copy(),
            prefill_len=self.prefill_len[pre].copy(),
            prefill_prefix=self.prefill_prefix[pre].copy(),
            block_table=self.block_table[rows].copy(),
            num_blocks=self.num_blocks,
        )


def _allocate_blocks(need: np.ndarray, rng: np.random.Generator, spare: int, max_blocks: int | None):
    num_blocks = int(need.sum()) + int(spare)
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = int(max(need.max() if need.size else 1, 1)) if max_blocks is None else int(max_blocks)
    table = np.full((need.shape[0], width), -1, dtype=np.int32)
    off = 0
    for r, n in enumerate(need):
        n = int(n)
        table[r, :n] = perm[off : off + n]
        off += n
    return table, num_blocks


def batch_from_lengths(
    decode_ctx,
    prefill_len,
    prefill_prefix=None,
    *,
    seed: int = 0,
    spare_blocks: int = 4,
    max_blocks: int | None = None,
    block_size: int = BLOCK_SIZE,
    shuffle: bool = True,
) -> Batch:
    """Build a batch with a (shuffled or identity) block table for given lengths."""
    decode_ctx = np.asarray(decode_ctx, dtype=np.int32).reshape(-1)
    prefill_len = np.asarray(prefill_len, dtype=np.int32).reshape(-1)
    if prefill_prefix is None:
        prefill_prefix = np.zeros_like(prefill_len)
    prefill_prefix = np.asarray(prefill_prefix, dtype=np.int32).reshape(-1)
    total = np.concatenate(
        [decode_ctx.astype(np.int64) + 1, prefill_prefix.astype(np.int64) + prefill_len.astype(np.int64)]
    )
    need = (total + block_size - 1) // block_size
    if shuffle:
        table, nb = _allocate_blocks(need, _rng(seed, STREAM_BLOCKS), spare_blocks, max_blocks)
    else:
        nb = int(need.sum()) + int(spare_blocks)
        width = int(max(need.max() if need.size else 1, 1)) if max_blocks is None else int(max_blocks)
        table = np.full((need.shape[0], width), -1, dtype=np.int32)
        off = 0
        for r, n in enumerate(need):
            table[r, : int(n)] = np.arange(off, off + int(n), dtype=np.int32)
            off += int(n)
    return Batch(decode_ctx, prefill_len, prefill_prefix, table, nb)


def make_batch(workload: str | Workload, seed: int, *, spare_blocks: int = 4, prefill_len=None,
               shuffle: bool = True) -> Batch:
    """Seeded dense batch of a workload (decodes first, then prefill chunks)."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    rng = _rng(seed, STREAM_LENGTHS)
    if prefill_len is not None:
        pre = np.asarray(prefill_len, dtype=np.int32).reshape(-1)
    elif wl.prefill_fixed:
        pre = np.asarray(wl.prefill_fixed, dtype=np.int32)
    elif wl.prefill_lognormal:
        median, sigma, cap = wl.prefill_lognormal
        draw = int(round(math.exp(rng.normal(math.log(median), sigma))))
        pre = np.asarray([min(max(draw, 1), cap)], dtype=np.int32)
    else:
        pre = np.zeros(0, dtype=np.int32)
    n_dec = wl.n_decode_fixed if wl.n_decode_fixed is not None else wl.n_tokens - int(pre.sum())
    lo, hi = wl.decode_ctx_range
    dec = rng.integers(lo, hi + 1, size=n_dec).astype(np.int32)
    return batch_from_lengths(dec, pre, None, seed=seed, spare_blocks=spare_blocks,
                              block_size=wl.shape.block_size, shuffle=shuffle)


# --------------------------------------------------------------------------------------
# weights and hidden states
# --------------------------------------------------------------------------------------

WEIGHT_STD = 0.02


def make_weights(shape: Shape, seed: int, *, gain_jitter: float = 0.0, layer: int = 0) -> dict:
    """bf16 random-init weights of one layer, Linear layout [out, in].

    ``w_qkv`` rows are [q (n_q*d) | k (n_kv*d) | v (n_kv*d)]; ``w_gate_up`` rows are
    [gate (F) | up (F)]. Norm gains are 1.0, or 1 + N(0, gain_jitter) when jittered.
    MoE shapes: ``w_gate_up`` [E, 2F, H] and ``w_down`` [E, H, F] (one FFN per expert) and
    ``w_router`` [E, H] ~ N(0, 1/H).
    """
    rng = _rng(seed * 1000 + layer, STREAM_WEIGHTS)
    H, F = shape.hidden, shape.ffn

    def w(rows, cols):
        buf = rng.standard_normal((rows, cols), dtype=np.float32)
        buf *= np.float32(WEIGHT_STD)
        return f32_to_bf16_bits(buf)

    def gain():
        if gain_jitter:
            return f32_to_bf16_bits(1.0 + rng.standard_normal(H, dtype=np.float32) * np.float32(gain_jitter))
        return f32_to_bf16_bits(np.ones(H, np.float32))

    out = {}
    out["g_attn"] = gain()
    out["w_qkv"] = w(shape.qkv_rows, H)
    out["w_o"] = w(H, shape.q_width)
    out["g_ffn"] = gain()
    if shape.n_experts:
        # per expert a SwiGLU FFN; router rows N(0, 1/H), so logits of a unit-RMS h2 are ~N(0, 1)
        E = shape.n_experts
        out["w_gate_up"] = np.stack([w(2 * F, H) for _ in range(E)])
        out["w_down"] = np.stack([w(H, F) for _ in range(E)])
        buf = rng.standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / math.sqrt(H))
        out["w_router"] = f32_to_bf16_bits(buf)
    else:
        out["w_gate_up"] = w(2 * F, H)
        out["w_down"] = w(H, F)
    return out


def make_x(shape: Shape, n_tokens: int, seed: int) -> np.ndarray:
    """Input hidden states x ~ N(0, 1), bf16 bits [T, H]."""
    rng = _rng(seed, STREAM_X)
    return f32_to_bf16_bits(rng.standard_normal((n_tokens, shape.hidden), dtype=np.float32))


# --------------------------------------------------------------------------------------
# KV pool history: counter-based hash, bit-identical on host (numpy) and device (torch)
# --------------------------------------------------------------------------------------

_M32 = 0xFFFFFFFF
_IH_SD = math.sqrt(4.0 * (65536.0**2 - 1.0) / 12.0)  # std of a sum of 4 uniform 16-bit ints


def kv_std(shape: Shape) -> float:
    """Std of cached K/V entries: that of h @ W^T for unit-RMS h and N(0, 0.02^2) weights."""
    return WEIGHT_STD * math.sqrt(shape.hidden)


def _keys(seed: int, layer: int, kind: int):
    base = (int(seed) * 0x9E3779B1 + int(layer) * 0x85EBCA77 + int(kind) * 0xC2B2AE3D) & _M32
    return base, (base ^ 0x5BD1E995) & _M32


def _mul32(x, m: int, xp):
    """(x * m) mod 2^32 with every intermediate below 2^63 (x, m < 2^32)."""
    lo = x & 0xFFFF
    hi = x >> 16
    return ((lo * m) + (((hi * m) & 0xFFFF) << 16)) & _M32


def _mix32(x, xp):
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D, xp)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B, xp)
    x = x ^ (x >> 16)
    return x


def _kv_f32_from_counter(counter, k1: int, k2: int, scale: float, xp, to_f32):
    # counters past 2^32: the high word is mixed into the keys (a high word of 0 leaves
    # them as they are, so smaller pools keep their values)
    hi = counter >> 32
    lo = counter & _M32
    mh = _mix32(hi, xp)
    h1 = _mix32(lo ^ (k1 ^ mh), xp)
    h2 = _mix32(lo ^ (k2 ^ mh), xp)
    s = (h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16)  # in [0, 262140]
    return (to_f32(s) - 131070.0) * scale  # both steps exact or single-rounded in fp32


def _kv_scale(shape: Shape) -> np.float32:
    return np.float32(kv_std(shape) / _IH_SD)


def make_kv_pool_blocks(shape: Shape, blocks, seed: int, layer: int = 0):
    """History contents of the given physical blocks (host, numpy).

    Returns (K, V) as uint16 bf16 bits with shapes K [n, n_kv, d/32, BS, 32] (keys in
    32-dim column chunks, each chunk token-major) and V [n, n_kv, d, BS] (dim-major values).
    Element (block b, head g, token t, dim i) has the same value whichever layout holds it.
    """
    blocks = np.asarray(blocks, dtype=np.int64).reshape(-1)
    G, BS, D = shape.n_kv, shape.block_size, shape.head_dim
    per_block = G * BS * D
    idx = (blocks[:, None] * per_block + np.arange(per_block, dtype=np.int64)[None, :]).astype(np.uint64)
    scale = _kv_scale(shape)
    out = []
    for kind in (0, 1):
        k1, k2 = _keys(seed, layer, kind)
        vals = _kv_f32_from_counter(idx, np.uint64(k1), np.uint64(k2), scale, np,
                                    lambda s: s.astype(np.int64).astype(np.float32))
        bits = f32_to_bf16_bits(vals).reshape(blocks.shape[0], G, BS, D)
        out.append(bits)
    k_bits, v_bits = out
    ch = _k_chunk(D)
    k_bits = k_bits.reshape(blocks.shape[0], G, BS, D // ch, ch).transpose(0, 1, 3, 2, 4)
    return np.ascontiguousarray(k_bits), np.ascontiguousarray(v_bits.transpose(0, 1, 3, 2))


def make_kv_pool(shape: Shape, num_blocks: int, seed: int, layer: int = 0):
    """Whole pool on the host (numpy); use for small pools."""
    return make_kv_pool_blocks(shape, np.arange(num_blocks), seed, layer)


def make_kv_pool_torch(shape: Shape, num_blocks: int, seed: int, layer: int = 0, device="cpu",
                       chunk_blocks: int = 4096):
    """Whole pool as torch int16 tensors on ``device`` (bit-identical to make_kv_pool).

    K is [num_blocks, n_kv, d/32, BS, 32], V is [num_blocks, n_kv, d, BS].
    """
    import torch

    G, BS, D = shape.n_kv, shape.block_size, shape.head_dim
    per_block = G * BS * D
    ch = _k_chunk(D)
    K = torch.empty((num_blocks, G, D // ch, BS, ch), dtype=torch.int16, device=device)
    V = torch.empty((num_blocks, G, D, BS), dtype=torch.int16, device=device)
    scale = float(_kv_scale(shape))
    for kind, dst in ((0, K), (1, V)):
        k1, k2 = _keys(seed, layer, kind)
        for b0 in range(0, num_blocks, chunk_blocks):
            b1 = min(num_blocks, b0 + chunk_blocks)
            idx = torch.arange(b0 * per_block, b1 * per_block, dtype=torch.int64, device=device)
            vals = _kv_f32_from_counter(idx, k1, k2, torch.tensor(scale, dtype=torch.float32, device=device),
                                        torch, lambda s: s.to(torch.float32))
            bits = vals.to(torch.bfloat16).view(torch.int16).view(b1 - b0, G, BS, D)
            if kind == 0:
                dst[b0:b1].copy_(bits.view(b1 - b0, G, BS, D // ch, ch).permute(0, 1, 3, 2, 4))
            else:
                dst[b0:b1].copy_(bits.transpose(2, 3))
            del idx, vals, bits
    return K, V


# --------------------------------------------------------------------------------------
# Counter-based weights (for many-layer stacks): bit-identical on host and device
# --------------------------------------------------------------------------------------

WEIGHT_NAMES = ("g_attn", "w_qkv", "w_o", "g_ffn", "w_gate_up", "w_down", "w_router")


def _weight_shapes(shape: Shape) -> dict:
    """(rows, cols) of each matrix; an MoE shape's expert matrices stack E of them."""
    H, F, E = shape.hidden, shape.ffn, shape.n_experts
    out = {"w_qkv": (shape.qkv_rows, H), "w_o": (H, shape.q_width)}
    if E:
        out.update({"w_gate_up": (E * 2 * F, H), "w_down": (E * H, F), "w_router": (E, H)})
    else:
        out.update({"w_gate_up": (2 * F, H), "w_down": (H, F)})
    return out


def _weight_scale(shape: Shape = None, name: str = "") -> np.float32:
    std = 1.0 / math.sqrt(shape.hidden) if name == "w_router" else WEIGHT_STD
    return np.float32(std / _IH_SD)


def _weight_dims(shape: Shape, name: str, n_rows: int, n_cols: int):
    E = shape.n_experts
    if E and name == "w_gate_up":
        return (E, 2 * shape.ffn, n_cols)
    if E and name == "w_down":
        return (E, shape.hidden, n_cols)
    return (n_rows, n_cols)


def make_weights_counter(shape: Shape, seed: int, layer: int, rows=None, matrices=None) -> dict:
    """One layer's weights from the counter-based generator (host, numpy).

    Every entry is a scaled sum of four uniform 16-bit integers drawn from a hash of
    (seed, layer, matrix, element index): mean 0, std WEIGHT_STD (an approximately normal
    draw bounded at +-3.46 std; the MoE router: std 1/sqrt(H)), rounded to bf16. Gains are
    1.0. ``rows`` (optional dict name -> row indices of the flattened [rows, cols] matrix)
    draws only those rows; ``matrices`` limits the names drawn.
    """
    out = {}
    H = shape.hidden
    one = f32_to_bf16_bits(np.ones(H, np.float32))
    shapes = _weight_shapes(shape)
    for name in matrices or WEIGHT_NAMES:
        if name in ("g_attn", "g_ffn"):
            out[name] = one.copy()
            continue
        if name not in shapes:
            continue
        scale = _weight_scale(shape, name)
        n_rows, n_cols = shapes[name]
        r = np.arange(n_rows, dtype=np.int64) if rows is None or name not in rows else np.asarray(rows[name], np.int64)
        idx = (r[:, None] * n_cols + np.arange(n_cols, dtype=np.int64)[None, :]).astype(np.uint64)
        k1, k2 = _keys(seed, 1000 + layer, 10 + WEIGHT_NAMES.index(name))
        vals = _kv_f32_from_counter(idx, np.uint64(k1), np.uint64(k2), scale, np,
                                    lambda s: s.astype(np.int64).astype(np.float32))
        out[name] = f32_to_bf16_bits(vals).reshape(len(r), n_cols)
        if rows is None or name not in rows:
            out[name] = out[name].reshape(_weight_dims(shape, name, n_rows, n_cols))
    return out


def make_weights_counter_torch(shape: Shape, seed: int, layer: int, device="cpu", chunk: int = 1 << 24) -> dict:
    """make_weights_counter as torch int16 tensors (bf16 bits) on ``device`` (bit-identical)."""
    import torch

    out = {}
    H = shape.hidden
    shapes = _weight_shapes(shape)
    for name in WEIGHT_NAMES:
        if name in ("g_attn", "g_ffn"):
            out[name] = torch.full((H,), 0x3F80, dtype=torch.int16, device=device)  # bf16 1.0
            continue
        if name not in shapes:
            continue
        scale = float(_weight_scale(shape, name))
        n_rows, n_cols = shapes[name]
        n = n_rows * n_cols
        if n > 2**32:
            raise ValueError("matrix too large for the 32-bit element counter")
        dst = torch.empty(n, dtype=torch.int16, device=device)
        k1, k2 = _keys(seed, 1000 + layer, 10 + WEIGHT_NAMES.index(name))
        for e0 in range(0, n, chunk):
            e1 = min(n, e0 + chunk)
            idx = torch.arange(e0, e1, dtype=torch.int64, device=device)
            vals = _kv_f32_from_counter(idx, k1, k2, torch.tensor(scale, dtype=torch.float32, device=device),
                                        torch, lambda s: s.to(torch.float32))
            dst[e0:e1].copy_(vals.to(torch.bfloat16).view(torch.int16))
            del idx, vals
        out[name] = dst.view(_weight_dims(shape, name, n_rows, n_cols))
    return out
