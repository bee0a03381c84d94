"""ctypes binding of libnanoflow (the C ABI declared in include/nanoflow.h).

Argument marshalling only: every computation happens in the HIP library. Functions carry
the C names and raise :class:`NanoflowError` on a negative status. The library must be
built (``python -m nano_intra_overlap_amd.build``); loading fails loudly otherwise — there
is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnanoflow.so")

NF_OK = 0
NF_E_ARG = -1
NF_E_BLOCK_RANGE = -2
NF_E_BLOCK_TABLE_SHORT = -3
NF_E_SLOT_ALIAS = -4
NF_E_PLAN = -5
NF_E_CU_MASK = -6
NF_E_HIP = -7
NF_E_UNSUPPORTED = -8
NF_E_CAPACITY = -9
NF_E_IO = -10
STATUS_NAMES = {v: k for k, v in dict(globals()).items() if k.startswith("NF_E_") or k == "NF_OK"}

NF_CU_MASK_WORDS = 8
NF_OP_KQV, NF_OP_DECATTN, NF_OP_PFATTN, NF_OP_O, NF_OP_UGD, NF_OP_KINDS = range(6)
NF_STACK_PIPELINE, NF_STACK_GRAPH = 1, 2
OP_NAMES = ["KQV", "DECATTN", "PFATTN", "O", "UGD"]
(NF_K_DECODE_ATTN, NF_K_DECODE_COMBINE, NF_K_PREFILL_ATTN, NF_K_GEMM_KQV, NF_K_GEMM_O, NF_K_GEMM_UG, NF_K_GEMM_DOWN,
 NF_K_RMSNORM, NF_K_ROPE_KV, NF_K_MOE_ROUTE, NF_K_MOE_COMBINE, NF_K_CLASSES) = range(12)
KERNEL_CLASS_NAMES = ["decode_attn", "decode_combine", "prefill_attn", "gemm_kqv", "gemm_o", "gemm_ug_swiglu",
                      "gemm_down", "rmsnorm", "rope_kv_append", "moe_route", "moe_combine"]

_i32p = ctypes.POINTER(ctypes.c_int32)
_u32p = ctypes.POINTER(ctypes.c_uint32)


class nf_layer_cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32)]


class nf_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("g_attn", "w_qkv", "w_o", "g_ffn", "w_gate_up", "w_down", "w_router")]


class nf_batch_desc(ctypes.Structure):
    _fields_ = [("n_decode", ctypes.c_int32), ("decode_ctx_len", _i32p), ("n_prefill", ctypes.c_int32),
                ("prefill_len", _i32p), ("prefill_prefix_len", _i32p), ("block_table", _i32p),
                ("max_blocks", ctypes.c_int32), ("block_table_dev", _i32p)]


class nf_kv_pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("num_blocks", ctypes.c_int32)]


class nf_plan(ctypes.Structure):
    _fields_ = [("n_nano", ctypes.c_int32), ("bounds", _i32p), ("n_streams", ctypes.c_int32), ("cu_masks", _u32p),
                ("n_ops", ctypes.c_int32), ("op_kind", _i32p), ("op_nano", _i32p), ("op_stream", _i32p),
                ("decode_max_workgroups", ctypes.c_int32), ("op_lane", _i32p)]


class nf_kv_ranges(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("first", _i32p), ("n_tokens", _i32p), ("block_table", _i32p),
                ("max_blocks", ctypes.c_int32)]


class NanoflowError(RuntimeError):
    def __init__(self, status: int, message: str = ""):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


_LIB = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libnanoflow.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libnanoflow is not built ({p} missing); run python -m nano_intra_overlap_amd.build")
    lib = ctypes.CDLL(p)
    V, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "nf_version": (ctypes.c_char_p, []),
        "nf_ctx_create": (I, [ctypes.c_int, ctypes.POINTER(V)]),
        "nf_ctx_destroy": (None, [V]),
        "nf_last_error": (ctypes.c_char_p, [V]),
        "nf_batch_slots": (I, [ctypes.POINTER(nf_layer_cfg), ctypes.POINTER(nf_batch_desc), I, _i32p, _i32p,
                               ctypes.c_char_p, S]),
        "nf_plan_dependencies": (I, [ctypes.POINTER(nf_batch_desc), ctypes.POINTER(nf_plan), _i32p, I, _i32p, _i32p,
                                     ctypes.c_char_p, S]),
        "nf_layer_forward": (I, [V, ctypes.POINTER(nf_layer_cfg), ctypes.POINTER(nf_layer_weights), V, V,
                                 ctypes.POINTER(nf_batch_desc), ctypes.POINTER(nf_kv_pool), ctypes.POINTER(nf_plan),
                                 V]),
        "nf_stack_dependencies": (I, [ctypes.POINTER(nf_batch_desc), ctypes.POINTER(nf_plan), I, I, _i32p, I, _i32p,
                                      _i32p, _i32p, ctypes.c_char_p, S]),
        "nf_stack_forward": (I, [V, ctypes.POINTER(nf_layer_cfg), I, ctypes.POINTER(nf_layer_weights), V, V,
                                 ctypes.POINTER(nf_batch_desc), ctypes.POINTER(nf_kv_pool), ctypes.POINTER(nf_plan),
                                 I, V]),
        "nf_debug_buffer": (I, [V, I, ctypes.POINTER(V), ctypes.POINTER(S)]),
        "nf_kv_offload": (I, [V, ctypes.POINTER(nf_layer_cfg), ctypes.POINTER(nf_kv_pool),
                              ctypes.POINTER(nf_kv_ranges), V, V]),
        "nf_kv_reload": (I, [V, ctypes.POINTER(nf_layer_cfg), ctypes.POINTER(nf_kv_pool), ctypes.POINTER(nf_kv_ranges),
                             V, V]),
        "nf_op_moe_ffn": (I, [V, ctypes.POINTER(nf_layer_cfg), ctypes.POINTER(nf_layer_weights), V, V, V, I, V, V, V]),
        "nf_op_gemm": (I, [V, V, V, V, V, I, I, I, I, I, V]),
        "nf_op_gemm_noalloc": (I, [V, V, V, V, V, I, I, I, I, I, V]),
        "nf_gemm_variants": (I, [_i32p, I, _i32p]),
        "nf_gemm_choice": (I, [I, I, I, I, _i32p, _i32p]),
        "nf_op_rmsnorm": (I, [V, V, V, V, I, I, ctypes.c_float, V]),
        "nf_op_rope_kv_append": (I, [V, ctypes.POINTER(nf_layer_cfg), V, ctypes.POINTER(nf_batch_desc),
                                     ctypes.POINTER(nf_kv_pool), V]),
        "nf_op_decode_attn": (I, [V, ctypes.POINTER(nf_layer_cfg), V, ctypes.POINTER(nf_batch_desc),
                                  ctypes.POINTER(nf_kv_pool), V, I, V]),
        "nf_op_prefill_attn": (I, [V, ctypes.POINTER(nf_layer_cfg), V, ctypes.POINTER(nf_batch_desc),
                                   ctypes.POINTER(nf_kv_pool), V, V]),
        "nf_profile_ops": (I, [V, ctypes.POINTER(nf_layer_cfg), ctypes.POINTER(nf_batch_desc), I, I, I,
                               ctypes.c_char_p]),
        "nf_profile_interference": (I, [V, ctypes.POINTER(nf_layer_cfg), ctypes.POINTER(nf_batch_desc), I,
                                        ctypes.POINTER(ctypes.c_float), I, ctypes.c_char_p]),
        "nf_plan_search": (I, [ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(nf_batch_desc), I, I,
                               ctypes.c_char_p, S]),
        "nf_ctx_set_timing": (I, [V, ctypes.c_uint32]),
        "nf_timing_summary": (I, [V, I, _i32p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double)]),
        "nf_ctx_set_decode_split": (I, [V, I]),
        "nf_ctx_set_prefill_chunk": (I, [V, I]),
        "nf_ctx_set_gemm_variant": (I, [V, I, I, I]),
        "nf_ctx_set_decode_launch": (I, [V, I, I, I]),
        "nf_copy_reference": (I, [V, V, S, V]),
        "nf_ctx_graph_stats": (I, [V, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    }
    missing = []
    for name, (res, args) in sig.items():
        try:
            fn = getattr(lib, name)
        except AttributeError:
            missing.append(name)
            continue
        fn.restype = res
        fn.argtypes = args
    if missing:
        raise ImportError(f"libnanoflow at {p} lacks symbols: {missing}")
    if path is None:
        _LIB = lib
    return lib


def _check(status: int, ctx=None, msg: str = ""):
    if status != NF_OK:
        if ctx is not None and not msg:
            msg = (load().nf_last_error(ctx) or b"").decode()
        raise NanoflowError(status, msg)


# ---------------------------------------------------------------------------------------
# host-side marshalling helpers
# ---------------------------------------------------------------------------------------


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(_i32p)


def make_cfg(shape) -> nf_layer_cfg:
    """nf_layer_cfg from any object with hidden, n_q, n_kv, head_dim, ffn, block_size, rms_eps, rope_base
    (and n_experts, top_k for MoE shapes)."""
    return nf_layer_cfg(shape.hidden, shape.n_q, shape.n_kv, shape.head_dim, shape.ffn, shape.block_size,
                        shape.rms_eps, shape.rope_base, getattr(shape, "n_experts", 0), getattr(shape, "top_k", 0))


class HostBatch:
    """nf_batch_desc over numpy arrays kept alive by this object."""

    def __init__(self, decode_ctx, prefill_len, prefill_prefix, block_table, block_table_dev_ptr: int | None = None):
        self.decode_ctx = _i32(decode_ctx).reshape(-1)
        self.prefill_len = _i32(prefill_len).reshape(-1)
        self.prefill_prefix = None if prefill_prefix is None else _i32(prefill_prefix).reshape(-1)
        self.block_table = _i32(block_table)
        if self.block_table.ndim != 2:
            raise ValueError("block_table must be 2-D [n_req, max_blocks]")
        self.desc = nf_batch_desc(
            self.decode_ctx.shape[0], _ptr(self.decode_ctx), self.prefill_len.shape[0], _ptr(self.prefill_len),
            _ptr(self.prefill_prefix), _ptr(self.block_table), self.block_table.shape[1],
            ctypes.cast(ctypes.c_void_p(block_table_dev_ptr), _i32p) if block_table_dev_ptr else None)

    @classmethod
    def from_batch(cls, b, block_table_dev_ptr: int | None = None) -> "HostBatch":
        return cls(b.decode_ctx, b.prefill_len, b.prefill_prefix, b.block_table, block_table_dev_ptr)

    @property
    def n_tokens(self) -> int:
        return int(self.decode_ctx.shape[0] + self.prefill_len.sum())


class HostPlan:
    """nf_plan over numpy arrays kept alive by this object.

    ops: list of (kind, nano, stream) in issue order; cu_masks: list of n_streams lists of
    NF_CU_MASK_WORDS words, or None for unmasked streams; lanes: None (lane = stream) or
    one lane (0..2) per listed op.
    """

    def __init__(self, bounds, ops, n_streams: int, cu_masks=None, decode_max_workgroups: int = 0, lanes=None):
        self.bounds = _i32(bounds)
        ops = np.asarray(ops, dtype=np.int32).reshape(-1, 3)
        self.kind = np.ascontiguousarray(ops[:, 0])
        self.nano = np.ascontiguousarray(ops[:, 1])
        self.stream = np.ascontiguousarray(ops[:, 2])
        self.lane = None if lanes is None else _i32(lanes)
        if self.lane is not None and self.lane.shape[0] != ops.shape[0]:
            raise ValueError("lanes needs one entry per op")
        self.masks = None
        if cu_masks is not None:
            self.masks = np.ascontiguousarray(np.asarray(cu_masks, dtype=np.uint32).reshape(n_streams, NF_CU_MASK_WORDS))
        self.n_streams = n_streams
        self.desc = nf_plan(self.bounds.shape[0] - 1, _ptr(self.bounds), n_streams,
                            None if self.masks is None else self.masks.ctypes.data_as(_u32p), ops.shape[0],
                            _ptr(self.kind), _ptr(self.nano), _ptr(self.stream), int(decode_max_workgroups),
                            None if self.lane is None else _ptr(self.lane))

    @property
    def ops(self):
        return list(zip(self.kind.tolist(), self.nano.tolist(), self.stream.tolist()))

    @property
    def lanes(self):
        return self.stream.tolist() if self.lane is None else self.lane.tolist()


def cu_mask(fraction: float | None = None, per_xcd: int | None = None, offset: int = 0, n_cu: int = 256):
    """A CU mask giving every XCD the same number of CUs.

    Bit i of the mask selects a CU of XCD i mod 8, so the bits [8*offset, 8*(offset+k))
    give each XCD k CUs. Either ``per_xcd`` (CUs per XCD) or ``fraction`` of the CUs.
    """
    per = n_cu // 8
    k = per_xcd if per_xcd is not None else max(1, min(per, int(round(fraction * per))))
    if not (1 <= k and offset >= 0 and offset + k <= per):
        raise ValueError("mask must give each XCD between 1 and 32 CUs")
    words = [0] * NF_CU_MASK_WORDS
    for i in range(8 * offset, 8 * (offset + k)):
        words[i // 32] |= 1 << (i % 32)
    return words


# ---------------------------------------------------------------------------------------
# C functions (same names)
# ---------------------------------------------------------------------------------------


def nf_version() -> str:
    return load().nf_version().decode()


def nf_ctx_create(device: int = 0):
    h = ctypes.c_void_p()
    _check(load().nf_ctx_create(device, ctypes.byref(h)), msg=f"device {device}")
    return h


def nf_ctx_destroy(ctx) -> None:
    load().nf_ctx_destroy(ctx)


def nf_last_error(ctx) -> str:
    return (load().nf_last_error(ctx) or b"").decode()


def nf_batch_slots(cfg: nf_layer_cfg, batch: HostBatch, num_blocks: int):
    """(positions, slots) per token; raises NanoflowError with the library's message."""
    T = batch.n_tokens
    pos = np.zeros(max(T, 1), np.int32)
    slot = np.zeros(max(T, 1), np.int32)
    err = ctypes.create_string_buffer(512)
    st = load().nf_batch_slots(ctypes.byref(cfg), ctypes.byref(batch.desc), num_blocks, _ptr(pos), _ptr(slot), err,
                               512)
    _check(st, msg=err.value.decode())
    return pos[:T], slot[:T]


def nf_plan_dependencies(batch: HostBatch, plan: HostPlan | None):
    """(edges [(i, j): op j depends on op i], global issue order)."""
    n_ops = len(plan.ops) if plan is not None else NF_OP_KINDS
    cap = n_ops * n_ops
    edges = np.zeros(2 * cap, np.int32)
    n = ctypes.c_int32()
    order = np.zeros(n_ops, np.int32)
    err = ctypes.create_string_buffer(512)
    st = load().nf_plan_dependencies(ctypes.byref(batch.desc), ctypes.byref(plan.desc) if plan else None,
                                     _ptr(edges), cap, ctypes.byref(n), _ptr(order), err, 512)
    _check(st, msg=err.value.decode())
    e = edges[: 2 * n.value].reshape(-1, 2)
    return [tuple(map(int, p)) for p in e], order.tolist()


def nf_layer_forward(ctx, cfg: nf_layer_cfg, weights: nf_layer_weights, x_ptr: int, y_ptr: int, batch: HostBatch,
                     pool: nf_kv_pool, plan: HostPlan | None, stream: int) -> None:
    st = load().nf_layer_forward(ctx, ctypes.byref(cfg), ctypes.byref(weights), x_ptr, y_ptr, ctypes.byref(batch.desc),
                                 ctypes.byref(pool), ctypes.byref(plan.desc) if plan is not None else None, stream)
    _check(st, ctx)


def nf_stack_dependencies(batch: HostBatch, plan: HostPlan | None, n_layers: int, flags: int = 0):
    """(edges [(i, j): stack op j depends on stack op i], listing, global issue order) of
    n_layers layers with one plan; stack op l * n_ops + i is the plan's op i in layer l."""
    n_ops = (len(plan.ops) if plan is not None else NF_OP_KINDS) * n_layers
    cap = n_ops * 8 + 64
    edges = np.zeros(2 * cap, np.int32)
    n = ctypes.c_int32()
    listing = np.zeros(n_ops, np.int32)
    order = np.zeros(n_ops, np.int32)
    err = ctypes.create_string_buffer(512)
    lib = load()
    st = lib.nf_stack_dependencies(ctypes.byref(batch.desc), ctypes.byref(plan.desc) if plan else None, n_layers,
                                   flags, _ptr(edges), cap, ctypes.byref(n), _ptr(listing), _ptr(order), err, 512)
    if st == NF_E_CAPACITY:
        cap = n.value
        edges = np.zeros(2 * cap, np.int32)
        st = lib.nf_stack_dependencies(ctypes.byref(batch.desc), ctypes.byref(plan.desc) if plan else None, n_layers,
                                       flags, _ptr(edges), cap, ctypes.byref(n), _ptr(listing), _ptr(order), err, 512)
    _check(st, msg=err.value.decode())
    e = edges[: 2 * n.value].reshape(-1, 2)
    return [tuple(map(int, p)) for p in e], listing.tolist(), order.tolist()


def nf_stack_forward(ctx, cfg: nf_layer_cfg, weights, x_ptr: int, y_ptr: int, batch: HostBatch, pools,
                     plan: HostPlan | None, flags: int, stream: int) -> None:
    """n_layers = len(weights) layers end to end; weights: nf_layer_weights per layer,
    pools: nf_kv_pool per layer."""
    n = len(weights)
    if len(pools) != n:
        raise ValueError("one pool per layer")
    w_arr = (nf_layer_weights * n)(*weights)
    p_arr = (nf_kv_pool * n)(*pools)
    st = load().nf_stack_forward(ctx, ctypes.byref(cfg), n, w_arr, x_ptr, y_ptr, ctypes.byref(batch.desc), p_arr,
                                 ctypes.byref(plan.desc) if plan is not None else None, flags, stream)
    _check(st, ctx)


def nf_debug_buffer(ctx, which: int):
    p = ctypes.c_void_p()
    n = ctypes.c_size_t()
    _check(load().nf_debug_buffer(ctx, which, ctypes.byref(p), ctypes.byref(n)), ctx)
    return p.value, n.value


def nf_op_gemm(ctx, A: int, B: int, C: int, R: int | None, m: int, n: int, k: int, epilogue: int = 0,
               variant: int = -1, stream: int = 0) -> None:
    _check(load().nf_op_gemm(ctx, A, B, C, R, m, n, k, epilogue, variant, stream), ctx)


def nf_op_gemm_noalloc(ctx, A: int, B: int, C: int, R: int | None, m: int, n: int, k: int, epilogue: int = 0,
                       variant: int = -1, stream: int = 0) -> None:
    """nf_op_gemm without any allocation (split-K partials in the library's static scratch)."""
    _check(load().nf_op_gemm_noalloc(ctx, A, B, C, R, m, n, k, epilogue, variant, stream), ctx)


class HostKvRanges:
    """Host arrays behind an nf_kv_ranges (kept alive with it)."""

    def __init__(self, first, n_tokens, block_table):
        self.first = _i32(first)
        self.n_tokens = _i32(n_tokens)
        self.block_table = _i32(np.asarray(block_table).reshape(len(self.first), -1))
        self.desc = nf_kv_ranges(len(self.first), _ptr(self.first), _ptr(self.n_tokens), _ptr(self.block_table),
                                 self.block_table.shape[1])

    @property
    def n_rows(self) -> int:
        return int(self.n_tokens.sum())


def nf_kv_offload(ctx, cfg: nf_layer_cfg, pool: nf_kv_pool, ranges: HostKvRanges, host_dst: int, stream: int = 0):
    _check(load().nf_kv_offload(ctx, ctypes.byref(cfg), ctypes.byref(pool), ctypes.byref(ranges.desc), host_dst,
                                stream), ctx)


def nf_kv_reload(ctx, cfg: nf_layer_cfg, pool: nf_kv_pool, ranges: HostKvRanges, host_src: int, stream: int = 0):
    _check(load().nf_kv_reload(ctx, ctypes.byref(cfg), ctypes.byref(pool), ctypes.byref(ranges.desc), host_src,
                               stream), ctx)


def nf_op_moe_ffn(ctx, cfg: nf_layer_cfg, weights: nf_layer_weights, h2: int, x1: int, y: int, n_tokens: int,
                  sel_out: int | None = None, wts_out: int | None = None, stream: int = 0) -> None:
    _check(load().nf_op_moe_ffn(ctx, ctypes.byref(cfg), ctypes.byref(weights), h2, x1, y, n_tokens, sel_out, wts_out,
                                stream), ctx)


def nf_gemm_variants():
    lib = load()
    cnt = ctypes.c_int32()
    _check(lib.nf_gemm_variants(ctypes.byref(cnt), 0, None))
    out = []
    for i in range(cnt.value):
        t = (ctypes.c_int32 * 5)()
        _check(lib.nf_gemm_variants(None, i, t))
        out.append(tuple(t))
    return out


def nf_gemm_choice(m: int, n: int, k: int, epilogue: int):
    """(variant, supported): the library's tile choice for nf_op_gemm at this shape (host)."""
    v, ok = ctypes.c_int32(), ctypes.c_int32()
    _check(load().nf_gemm_choice(m, n, k, epilogue, ctypes.byref(v), ctypes.byref(ok)))
    return v.value, bool(ok.value)


def nf_op_rmsnorm(ctx, x: int, g: int, out: int, m: int, n: int, eps: float, stream: int = 0) -> None:
    _check(load().nf_op_rmsnorm(ctx, x, g, out, m, n, eps, stream), ctx)


def nf_op_rope_kv_append(ctx, cfg: nf_layer_cfg, qkv: int, batch: HostBatch, pool: nf_kv_pool, stream: int = 0):
    _check(load().nf_op_rope_kv_append(ctx, ctypes.byref(cfg), qkv, ctypes.byref(batch.desc), ctypes.byref(pool),
                                       stream), ctx)


def nf_op_decode_attn(ctx, cfg: nf_layer_cfg, qkv: int, batch: HostBatch, pool: nf_kv_pool, out: int,
                      kv_split_blocks: int = 0, stream: int = 0) -> None:
    _check(load().nf_op_decode_attn(ctx, ctypes.byref(cfg), qkv, ctypes.byref(batch.desc), ctypes.byref(pool), out,
                                    kv_split_blocks, stream), ctx)


def nf_op_prefill_attn(ctx, cfg: nf_layer_cfg, qkv: int, batch: HostBatch, pool: nf_kv_pool, out: int,
                       stream: int = 0) -> None:
    _check(load().nf_op_prefill_attn(ctx, ctypes.byref(cfg), qkv, ctypes.byref(batch.desc), ctypes.byref(pool), out,
                                     stream), ctx)


def nf_profile_ops(ctx, cfg: nf_layer_cfg, batch: HostBatch, num_blocks: int, step: int, max_tokens: int,
                   out_json: str) -> None:
    _check(load().nf_profile_ops(ctx, ctypes.byref(cfg), ctypes.byref(batch.desc), num_blocks, step, max_tokens,
                                 out_json.encode()), ctx)


def nf_profile_interference(ctx, cfg: nf_layer_cfg, batch: HostBatch, num_blocks: int, r_grid, out_json: str) -> None:
    arr = (ctypes.c_float * len(r_grid))(*r_grid)
    _check(load().nf_profile_interference(ctx, ctypes.byref(cfg), ctypes.byref(batch.desc), num_blocks, arr,
                                          len(r_grid), out_json.encode()), ctx)


def nf_plan_search(dbest_json: str, rp_json: str, batch: HostBatch, max_nano: int = 4, granularity: int = 128,
                   cap: int = 1 << 16) -> str:
    buf = ctypes.create_string_buffer(cap)
    st = load().nf_plan_search(dbest_json.encode(), rp_json.encode(), ctypes.byref(batch.desc), max_nano, granularity,
                               buf, cap)
    if st != NF_OK:
        raise NanoflowError(st, buf.value.decode())
    return buf.value.decode()


def nf_copy_reference(dst: int, src: int, nbytes: int, stream: int = 0) -> None:
    """Known-size device copy (reference for hardware traffic counters)."""
    st = load().nf_copy_reference(dst, src, nbytes, stream)
    if st != NF_OK:
        raise NanoflowError(st, "nf_copy_reference failed")


def nf_ctx_set_timing(ctx, class_mask: int) -> None:
    _check(load().nf_ctx_set_timing(ctx, class_mask), ctx)


def nf_timing_summary(ctx, cls: int):
    """(count, total_ms, min_ms, max_ms) of the timed launches of a kernel class."""
    n = ctypes.c_int32()
    tot, mn, mx = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(load().nf_timing_summary(ctx, cls, ctypes.byref(n), ctypes.byref(tot), ctypes.byref(mn), ctypes.byref(mx)),
           ctx)
    return n.value, tot.value, mn.value, mx.value


def nf_ctx_set_decode_split(ctx, blocks: int) -> None:
    _check(load().nf_ctx_set_decode_split(ctx, blocks), ctx)


def nf_ctx_set_prefill_chunk(ctx, keys: int) -> None:
    """Prefill attention keys per work item (0 = the library's choice per nano-op)."""
    _check(load().nf_ctx_set_prefill_chunk(ctx, keys), ctx)


def nf_ctx_set_decode_launch(ctx, max_workgroups: int, nbuf: int = 0, ring: int = 0) -> None:
    """Decode attention launch: workgroup cap (0 = one wave per unit), KV blocks per softmax
    step, and ring depth (register buffers of nbuf blocks; ring - 1 groups in flight);
    nbuf = ring = 0 lets each launch choose from its work (the default)."""
    _check(load().nf_ctx_set_decode_launch(ctx, max_workgroups, nbuf, ring), ctx)


def nf_ctx_graph_stats(ctx):
    """(captures, launches) of the context's layer-stack graph so far."""
    c, n = ctypes.c_int64(), ctypes.c_int64()
    _check(load().nf_ctx_graph_stats(ctx, ctypes.byref(c), ctypes.byref(n)), ctx)
    return c.value, n.value


def nf_ctx_set_gemm_variant(ctx, kind: int, which: int, variant: int) -> None:
    _check(load().nf_ctx_set_gemm_variant(ctx, kind, which, variant), ctx)
