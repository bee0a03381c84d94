#!/usr/bin/env python3
"""Benchmark of one nano-batched decoder-layer iteration on one MI355X.

A step is one nf_layer_forward call over the dense batch (host batch layout and slot
derivation, metadata upload, then every nano-operation: RMSNorm, KQV GEMM, rotary + KV
append, decode and prefill attention, O GEMM + residual, RMSNorm, Up/Gate GEMM + SwiGLU,
Down GEMM + residual), with weights, activations, KV pool and block table resident in HBM
before the timed region starts. For a layer-stack workload (the 32-layer 8B stack) a step
is one nf_stack_forward call: every layer end to end over the batch, each layer with its
own weights and KV pool.

Prints one JSON line: tokens/s, the dominant kernel's roofline (live HIP-event timing on
the stream it runs on), the fraction of the bf16 MFMA peak the layer reaches, the
sequential single-stream baseline, and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "tokens/s/GPU at 2048-token dense batch; % of bf16 MFMA roofline"
PEAK_BF16 = 2.5e15  # dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12  # HBM3E, B/s


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama3_8b_layer")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--prefill-len", type=int, default=0,
                   help="one prefill chunk of this many tokens instead of the workload's draw (the rest decode)")
    p.add_argument("--plan", default="searched", choices=["overlap", "sequential", "null", "searched"],
                   help="searched: the two-stage search's plan for this batch (from the profiled tables)")
    p.add_argument("--n-nano", type=int, default=2)
    p.add_argument("--mem-cus", type=int, default=0, help="CUs per XCD for the memory stream (0 = unmasked)")
    p.add_argument("--plan-json", default="", help="plan written by nf_plan_search (with --plan searched)")
    p.add_argument("--no-baseline", action="store_true",
                   help="skip the comparison schedules (sequential, nano-batching only, overlap template)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-decode-sample", type=int, default=-1,
                   help="decode requests in the CPU oracle's sample (-1 = all: the whole dense batch)")
    p.add_argument("--decode-grid", type=int, default=0, help="max decode-attention workgroups (0 = one wave per unit)")
    p.add_argument("--decode-split", type=int, default=0,
                   help="decode split-KV chunk in KV blocks (0 = the library's choice per nano-op)")
    p.add_argument("--prefill-chunk", type=int, default=0,
                   help="prefill attention keys per work item (0 = the library's choice)")
    p.add_argument("--decode-nbuf", type=int, default=0, choices=[0, 1, 2],
                   help="KV blocks per softmax step (0 with --decode-ring 0: chosen per launch)")
    p.add_argument("--decode-ring", type=int, default=0, choices=[0, 2, 3, 4],
                   help="decode attention register ring depth (ring - 1 groups of KV blocks in flight)")
    p.add_argument("--gemm-variant", type=int, default=-1, help="force one GEMM tile variant for every GEMM")
    p.add_argument("--gemm-variants", default="",
                   help="tile variants of the KQV, O, Up/Gate and Down GEMMs, comma-separated (-1 = library choice)")
    p.add_argument("--no-pipeline", action="store_true",
                   help="layer stacks: issue layer by layer instead of cross-layer pipelining")
    p.add_argument("--cpu-layers", type=int, default=2,
                   help="layer stacks: layers the CPU oracle runs on its sample (its time is scaled to all layers)")
    p.add_argument("--kv-io", action="store_true",
                   help="also measure KV offload / multi-round reload (adds a kv_io object to the JSON line)")
    p.add_argument("--vendor-gemm", action="store_true",
                   help="also time the layer's four dense products alone, this library's GEMM against the "
                        "vendor library's (torch.nn.functional.linear, hipBLASLt), into gemm_vs_vendor")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB first (a known-size reference for "
                        "hardware traffic counters)")
    return p.parse_args()


def gemm_vs_vendor(ctx, shape, T: int, seed: int) -> dict:
    """The layer's dense products at T rows, each alone and back to back: nf_op_gemm (library
    tile choice, fused epilogue) against torch.nn.functional.linear (the vendor library's
    plain product). Best of 3 x 30 launches timed with events on torch's current stream; a
    comparison only, nothing of the layer runs through the vendor library."""
    import torch

    from nano_intra_overlap_amd import abi

    g = torch.Generator(device="cuda").manual_seed(seed)
    prods = {"kqv": (shape.qkv_rows, shape.hidden, 0), "o": (shape.hidden, shape.q_width, 1),
             "ug_swiglu": (shape.ffn, shape.hidden, 2), "down": (shape.hidden, shape.ffn, 1)}
    stream = torch.cuda.current_stream()

    def best_us(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(30):
                fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 30 * 1e3)
        return best

    res = {}
    for name, (n, k, epi) in prods.items():
        nb = 2 * n if epi == 2 else n
        A = (torch.randn(T, k, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
        B = (torch.randn(nb, k, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
        R = torch.randn(T, n, device="cuda", generator=g).to(torch.bfloat16)
        C = torch.empty(T, n, device="cuda", dtype=torch.bfloat16)
        ours = best_us(lambda: abi.nf_op_gemm(ctx, A.data_ptr(), B.data_ptr(), C.data_ptr(), R.data_ptr(), T, n, k,
                                              epi, -1, stream.cuda_stream))
        vendor = best_us(lambda: torch.nn.functional.linear(A, B))
        flops = 2.0 * T * nb * k
        res[name] = {"m": T, "n": nb, "k": k, "variant": abi.nf_gemm_choice(T, n, k, epi)[0],
                     "ours_us": round(ours, 1), "vendor_us": round(vendor, 1),
                     "ours_tflops": round(flops / ours / 1e6, 1), "vendor_tflops": round(flops / vendor / 1e6, 1)}
        print(f"[bench] {name}: ours {ours:.1f} us, vendor {vendor:.1f} us (plain product)", file=sys.stderr,
              flush=True)
        del A, B, R, C
    return res


def kernel_source_hash(files) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(workload: str, seed: int, launches_per_step: float):
    """HBM bytes per decode-attention launch from the committed hardware-counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a known-size copy),
    or None when there is none for this workload and launch count, or when the kernel's
    source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"decode_attn_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if (rec.get("seed") != seed or rec.get("decode_launches_per_step") != launches_per_step
            or rec.get("source_sha256") != kernel_source_hash(rec["source_files"])):
        return None
    return int(rec["traffic_bytes_per_launch"])


def algorithmic(shape, b, n_nano):
    """Algorithmic FLOPs and bytes of one layer iteration (per-unit figures x units)."""
    H, nq, nkv, d, F = shape.hidden, shape.n_q, shape.n_kv, shape.head_dim, shape.ffn
    T = b.n_tokens
    E, k = shape.n_experts, (shape.top_k if shape.n_experts else 1)
    p_attn = H * (nq + 2 * nkv) * d + nq * d * H
    # weight elements a token multiplies (MoE: its top_k experts and the router)
    p_layer = p_attn + k * 3 * H * F + E * H
    gemm_flops = 2 * T * p_layer
    ctx = b.decode_ctx.astype(np.int64)
    kv_unit = 2 * nkv * d * 2  # bytes of K and V per key (all KV heads)
    decode_keys = int((ctx + 1).sum())
    decode_bytes = decode_keys * kv_unit + b.n_decode * (nq * d * 2) * 2  # KV stream + q in + o out
    pre = b.prefill_len.astype(np.int64)
    attn_flops = 4 * d * nq * (decode_keys + int((pre * (pre + 1) // 2).sum()))
    weight_bytes = 2 * (p_attn + max(E, 1) * 3 * H * F + E * H)  # every weight read once
    act_bytes = T * H * 2 * 2 + T * 2 * nkv * d * 2  # x in, y out, new K/V written
    return {
        "gemm_flops": gemm_flops,
        "attn_flops": attn_flops,
        "decode_bytes": decode_bytes,
        "decode_keys": decode_keys,
        "kv_unit_bytes": kv_unit,
        "layer_bytes": decode_bytes + int(pre.sum()) * kv_unit + n_nano * weight_bytes + act_bytes,
        "p_layer": p_layer,
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(shape, b, ws, x, seed, n_dec, fetch_blocks, n_layers_total=1, repeats=3):
    """The oracle as it stands, timed on a sample of the workload: n_dec decode requests
    (all of them when n_dec < 0) plus every prefill chunk, over a compact copy of the KV
    blocks they use (fetch_blocks(layer, ids) -> (k, v) bf16 bit arrays of those pool
    blocks), through the layers of ``ws`` (host weight dicts): one warm-up pass, then the
    median of ``repeats`` timed passes; the time is scaled to n_layers_total layers."""
    from oracle import layer as ol
    from synth import workloads as sw

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    if n_dec < 0 or n_dec >= b.n_decode:
        n_dec = b.n_decode
        sample = list(range(b.n_requests))
    else:
        rng = np.random.default_rng(seed + 7)
        sample = sorted(rng.choice(b.n_decode, size=n_dec, replace=False).tolist()) + list(
            range(b.n_decode, b.n_requests))
    sub = b.select(sample)
    ranges = ol.request_ranges(b)
    rows = np.concatenate([np.arange(ranges[r][0], ranges[r][1]) for r in sample])
    need = (sub.cached_lens() + sub.q_lens() + 15) // 16
    mask = np.arange(sub.block_table.shape[1])[None, :] < need[:, None]
    used = np.unique(sub.block_table[mask])
    bt = np.full_like(sub.block_table, -1)
    bt[mask] = np.searchsorted(used, sub.block_table[mask])
    compact = sw.Batch(sub.decode_ctx, sub.prefill_len, sub.prefill_prefix, bt, len(used))
    pools = [fetch_blocks(l, used) for l in range(len(ws))]
    xs = x[rows]
    times = []
    for rep in range(1 + repeats):  # one warm-up pass, then the timed ones
        t0 = time.perf_counter()
        ol.stack_forward(shape, ws, xs, compact, [p[0] for p in pools], [p[1] for p in pools])
        if rep:
            times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    dt_all = dt * n_layers_total / len(ws)
    what = ("the whole dense batch" if n_dec == b.n_decode else
            f"{n_dec} of {b.n_decode} decode requests (sampled, seed {seed + 7}) + all prefill chunks")
    spread = f"median of {repeats} after a warm-up pass; passes {min(times):.2f}-{max(times):.2f} s"
    layers = (f"one float64 layer pass in {dt:.2f} s ({spread})" if n_layers_total == 1 else
              f"{len(ws)} of {n_layers_total} float64 layer passes in {dt:.2f} s ({spread}), scaled to all layers")
    return {
        "value": round(len(rows) / dt_all, 2),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what}: {len(rows)} tokens ({b.n_prefill} prefill chunk(s), {int(b.prefill_len.sum())} "
                  f"tokens), {len(used)} KV blocks; {layers} "
                  f"({cpu_model()}, {os.cpu_count()} host CPUs, {threads} BLAS threads)",
    }


def kv_io_probe(abi, torch, ctx, cfg, shape, b, step, stream, n_conv=16, conv_len=2048, steps=10):
    """KV movement measured on its own and beside the layer (summary page, "KV-cache
    management and offloading").

    reload: n_conv conversations of conv_len tokens each, from pinned host rows into a pool
    of their own (shuffled pages): the library's two-stage path (one contiguous copy in +
    the scatter kernel), a plain contiguous host-to-device copy of the same bytes, and
    per-page copies (one 4-KB copy per (block, KV head) of K and of V, issued from Python,
    first 2048 pieces) as the naive path the pages compare against.
    offload: the batch's new tokens (one row each) copied out after every layer step, on a
    second stream beside the next step, against steps without it."""
    from nano_intra_overlap_amd.device import DevicePool

    row_bytes = 2 * shape.n_kv * shape.head_dim * 2
    n_tok = n_conv * conv_len
    nb = n_tok // 16
    rng = np.random.default_rng(5)
    table = rng.permutation(nb).astype(np.int32).reshape(n_conv, conv_len // 16)
    ranges = abi.HostKvRanges([0] * n_conv, [conv_len] * n_conv, table)
    k = torch.empty((nb, shape.n_kv, shape.head_dim // 32, 16, 32), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((nb, shape.n_kv, shape.head_dim, 16), dtype=torch.bfloat16, device="cuda")
    pool = DevicePool(k, v)
    host = torch.empty(n_tok * row_bytes // 2, dtype=torch.int16, pin_memory=True)
    host.numpy()[:] = rng.integers(-2000, 2000, host.shape[0], dtype=np.int16)
    dev = torch.empty(n_tok * row_bytes // 2, dtype=torch.int16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    nbytes = n_tok * row_bytes
    t_reload = timed(lambda: abi.nf_kv_reload(ctx, cfg, pool.desc, ranges, host.data_ptr(), stream))
    t_h2d = timed(lambda: dev.copy_(host, non_blocking=True))
    t_off = timed(lambda: abi.nf_kv_offload(ctx, cfg, pool.desc, ranges, host.data_ptr(), stream))
    # naive: one copy per (block, KV head) piece of K and of V, straight into the pages
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.restype = ctypes.c_int
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    piece = 16 * shape.head_dim * 2
    n_pieces = 2048

    def naive():
        base_k, base_v, src = k.data_ptr(), v.data_ptr(), host.data_ptr()
        for i in range(n_pieces // 2):
            blk, g = divmod(i, shape.n_kv)
            off = (blk * shape.n_kv + g) * piece
            hip.hipMemcpyAsync(base_k + off, src + 2 * i * piece, piece, 1, ctypes.c_void_p(stream))
            hip.hipMemcpyAsync(base_v + off, src + (2 * i + 1) * piece, piece, 1, ctypes.c_void_p(stream))

    t_naive = timed(naive, reps=3)
    # offload of every new token beside the layer
    new = abi.HostKvRanges(np.concatenate([b.decode_ctx, b.prefill_prefix]),
                           np.concatenate([np.ones(b.n_decode, np.int32), b.prefill_len]), b.block_table)
    out = torch.empty(new.n_rows * row_bytes // 2, dtype=torch.int16, pin_memory=True)
    side = torch.cuda.Stream()
    done = torch.cuda.Event()

    def step_with_offload():
        step()
        done.record()
        side.wait_event(done)
        abi.nf_kv_offload(ctx, cfg, step.pool_desc, new, out.data_ptr(), side.cuda_stream)

    t_plain = timed(step, reps=steps)
    t_with = timed(step_with_offload, reps=steps)
    torch.cuda.synchronize()
    return {
        "reload": {"conversations": n_conv, "tokens": n_tok, "bytes": nbytes, "ms": round(t_reload, 4),
                   "GB_per_s": round(nbytes / t_reload / 1e6, 1)},
        "contiguous_h2d": {"ms": round(t_h2d, 4), "GB_per_s": round(nbytes / t_h2d / 1e6, 1)},
        "scatter_share_ms": round(t_reload - t_h2d, 4),
        "naive_page_copies": {"pieces": n_pieces, "bytes_each": piece, "ms": round(t_naive, 4),
                              "GB_per_s": round(n_pieces * piece / t_naive / 1e6, 2),
                              "note": "one hipMemcpyAsync per (block, KV head) piece, issued from Python"},
        "offload_all": {"ms": round(t_off, 4), "GB_per_s": round(nbytes / t_off / 1e6, 1)},
        "layer_step_ms": round(t_plain, 4),
        "layer_step_with_offload_ms": round(t_with, 4),
        "offload_rows_per_step": new.n_rows,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from nano_intra_overlap_amd import abi, plans
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_tensor
    from synth import workloads as sw
    from synth.workloads import make_kv_pool_torch

    assert torch.cuda.is_available(), "bench needs a GPU"
    wl = sw.WORKLOADS[args.workload]
    shape = wl.shape
    b = sw.make_batch(args.workload, args.seed, prefill_len=[args.prefill_len] if args.prefill_len else None)
    T = b.n_tokens
    log(f"workload {wl.name}: T={T}, decode={b.n_decode}, prefill={b.prefill_len.tolist()}, blocks={b.num_blocks}")
    t0 = time.time()
    n_layers = shape.n_layers
    stack = n_layers > 1
    x = sw.make_x(shape, T, args.seed)
    xd = bf16_tensor(x, "cuda")
    yd = torch.empty_like(xd)
    if stack or shape.n_experts:
        # every layer's weights (counter-based generator, drawn on the device) and KV pool
        w = None
        wds = [DeviceWeights.from_int16(sw.make_weights_counter_torch(shape, args.seed, l, device="cuda"))
               for l in range(n_layers)]
        k16s, v16s = [], []
        for l in range(n_layers):
            k16, v16 = make_kv_pool_torch(shape, b.num_blocks, args.seed, layer=l, device="cuda")
            k16s.append(k16)
            v16s.append(v16)
        pools = [DevicePool.from_int16(k, v) for k, v in zip(k16s, v16s)]
    else:
        w = sw.make_weights(shape, args.seed)
        wds = [DeviceWeights(w, "cuda")]
        k16, v16 = make_kv_pool_torch(shape, b.num_blocks, args.seed, device="cuda")
        k16s, v16s = [k16], [v16]
        pools = [DevicePool.from_int16(k16, v16)]
    w_descs = [wd.desc for wd in wds]
    p_descs = [p.desc for p in pools]
    bt_dev = torch.from_numpy(np.ascontiguousarray(b.block_table)).cuda()
    hb = abi.HostBatch.from_batch(b, block_table_dev_ptr=bt_dev.data_ptr())
    cfg = abi.make_cfg(shape)
    torch.cuda.synchronize()
    free, total = torch.cuda.mem_get_info()
    log(f"inputs resident in {time.time() - t0:.1f} s ({n_layers} layer(s); device memory used "
        f"{(total - free) / 1e9:.1f} of {total / 1e9:.1f} GB)")

    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        abi.nf_copy_reference(dst.data_ptr(), src.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert bool((dst == 1).all()), "reference copy mismatch"
        log(f"reference copy: {nbytes} bytes read + {nbytes} bytes written (copy_ref_kernel)")
        del src, dst

    ctx = abi.nf_ctx_create(0)
    stream = torch.cuda.current_stream().cuda_stream
    abi.nf_ctx_set_decode_launch(ctx, args.decode_grid, args.decode_nbuf, args.decode_ring)
    if args.decode_split:
        abi.nf_ctx_set_decode_split(ctx, args.decode_split)
    if args.prefill_chunk:
        abi.nf_ctx_set_prefill_chunk(ctx, args.prefill_chunk)
    if args.gemm_variant >= 0:
        for kind in (abi.NF_OP_KQV, abi.NF_OP_O, abi.NF_OP_UGD):
            for which in (0, 1):
                abi.nf_ctx_set_gemm_variant(ctx, kind, which, args.gemm_variant)
    if args.gemm_variants:
        vs = [int(v) for v in args.gemm_variants.split(",")]
        if len(vs) != 4:
            raise SystemExit("--gemm-variants takes four variants: KQV,O,UG,Down")
        for (kind, which), v in zip(((abi.NF_OP_KQV, 0), (abi.NF_OP_O, 0), (abi.NF_OP_UGD, 0), (abi.NF_OP_UGD, 1)), vs):
            abi.nf_ctx_set_gemm_variant(ctx, kind, which, v)

    def make_plan(kind):
        if kind == "null":
            return None, "sequential, one nano-batch, caller stream"
        if kind == "sequential":
            bounds = plans.even_bounds(T, args.n_nano)
            return plans.sequential(hb, bounds), f"sequential, {len(bounds) - 1} nano-batches"
        if kind == "searched":
            from nano_intra_overlap_amd import autosearch

            text = open(args.plan_json).read() if args.plan_json else autosearch.search_plan(args.workload, args.seed)
            plan, rec = plans.from_json(text)
            return plan, f"searched: {rec.get('summary', '')}"
        bounds = plans.even_bounds(T, args.n_nano)
        masks = (None, None)
        if args.mem_cus:
            masks = (abi.cu_mask(per_xcd=32 - args.mem_cus, offset=0), abi.cu_mask(per_xcd=args.mem_cus,
                                                                                     offset=32 - args.mem_cus))
        desc = f"overlap, {len(bounds) - 1} nano-batches, bounds {bounds}, memory stream " + (
            f"{args.mem_cus}/32 CUs per XCD" if args.mem_cus else "unmasked")
        return plans.overlap(hb, bounds, *masks), desc

    stack_flags = 0 if args.no_pipeline else abi.NF_STACK_PIPELINE

    def step(plan, flags):
        if stack:
            abi.nf_stack_forward(ctx, cfg, w_descs, xd.data_ptr(), yd.data_ptr(), hb, p_descs, plan, flags, stream)
        else:
            abi.nf_layer_forward(ctx, cfg, w_descs[0], xd.data_ptr(), yd.data_ptr(), hb, p_descs[0], plan, stream)

    def run(plan, steps, warmup, timing_mask=0, flags=None):
        flags = stack_flags if flags is None else flags
        for _ in range(warmup):
            step(plan, flags)
        torch.cuda.synchronize()
        abi.nf_ctx_set_timing(ctx, timing_mask)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step(plan, flags)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        kernels = {}
        for cls in range(abi.NF_K_CLASSES):
            if timing_mask >> cls & 1:
                n, tot, mn, mx = abi.nf_timing_summary(ctx, cls)
                kernels[abi.KERNEL_CLASS_NAMES[cls]] = {"launches": n, "total_ms": tot, "min_ms": mn, "max_ms": mx}
        abi.nf_ctx_set_timing(ctx, 0)
        return ms, kernels

    plan, plan_desc = make_plan(args.plan)
    alg = algorithmic(shape, b, 1 if plan is None else len(plan.bounds) - 1)

    # timed region: the whole step, with the dominant kernel (decode attention) bracketed
    # by HIP events on its own stream
    ms, kern = run(plan, args.steps, args.warmup, 1 << abi.NF_K_DECODE_ATTN)
    dk = kern["decode_attn"]
    launches_per_step = dk["launches"] / args.steps
    dec_avg_ms = dk["total_ms"] / dk["launches"]
    bytes_per_launch = alg["decode_bytes"] * n_layers / launches_per_step
    achieved = bytes_per_launch / (dec_avg_ms * 1e-3)
    log(f"plan: {plan_desc}: {ms:.3f} ms/step; decode attention {dec_avg_ms:.3f} ms/launch "
        f"x {launches_per_step:g} -> {achieved / 1e9:.0f} GB/s")

    # step-time distribution (separate pass, one event pair per step; informational)
    for _ in range(2):
        step(plan, stack_flags)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, z in evs:
        a.record()
        step(plan, stack_flags)
        z.record()
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(z) for a, z in evs])
    dist = {q: round(float(np.percentile(per_step, p)), 4) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}

    # measured copy bandwidth on this GPU: nf_copy_reference reading and writing 1 GiB
    cbytes = 1 << 30
    csrc = torch.ones(cbytes // 2, dtype=torch.bfloat16, device="cuda")
    cdst = torch.empty_like(csrc)
    abi.nf_copy_reference(cdst.data_ptr(), csrc.data_ptr(), cbytes, stream)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        abi.nf_copy_reference(cdst.data_ptr(), csrc.data_ptr(), cbytes, stream)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * cbytes * 3 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst

    # per-kernel breakdown (separate instrumented pass; informational)
    all_mask = (1 << abi.NF_K_CLASSES) - 1
    _, breakdown = run(plan, 5, 1, all_mask)
    for k, v in breakdown.items():
        v["avg_ms"] = v["total_ms"] / max(v["launches"], 1)
    fan = shape.top_k if shape.n_experts else 1  # rows per token of the FFN products
    flops_by = {
        "gemm_kqv": 2 * T * shape.hidden * shape.qkv_rows,
        "gemm_o": 2 * T * shape.q_width * shape.hidden,
        "gemm_ug_swiglu": 2 * fan * T * shape.hidden * 2 * shape.ffn,
        "gemm_down": 2 * fan * T * shape.ffn * shape.hidden,
    }
    for k, f in flops_by.items():
        f *= n_layers
        if k in breakdown and breakdown[k]["launches"]:
            per_step_ms = breakdown[k]["total_ms"] / 5
            breakdown[k]["tflops"] = round(f / (per_step_ms * 1e-3) / 1e12, 1)
            breakdown[k]["mfma_frac"] = round(f / (per_step_ms * 1e-3) / PEAK_BF16, 4)

    own_peak = max((v.get("tflops", 0.0) for k, v in breakdown.items() if k.startswith("gemm")), default=0.0) or None
    # prefill attention: 4 d per (query head, causally visible key), as the oracle counts it
    pre, pfx = b.prefill_len.astype(np.int64), b.prefill_prefix.astype(np.int64)
    pf_flops = 4 * shape.head_dim * shape.n_q * int((pre * pfx + pre * (pre + 1) // 2).sum()) * n_layers
    if breakdown.get("prefill_attn", {}).get("launches"):
        per_step_ms = breakdown["prefill_attn"]["total_ms"] / 5
        breakdown["prefill_attn"]["tflops"] = round(pf_flops / (per_step_ms * 1e-3) / 1e12, 1)
        breakdown["prefill_attn"]["mfma_frac"] = round(pf_flops / (per_step_ms * 1e-3) / PEAK_BF16, 4)

    # comparison schedules on the same batch: the plain sequential layer (one nano-batch,
    # caller stream), nano-batching without overlap, and the two-stream overlap template
    schedules = {"timed": round(ms, 4)}
    seq_ms = None
    if not args.no_baseline:
        seq_ms, _ = run(None, args.steps, args.warmup, flags=0)
        schedules["sequential"] = round(seq_ms, 4)
        for n in (2, 4):
            bnd = plans.even_bounds(T, n)
            schedules[f"nanobatch_only_{n}"] = round(run(plans.sequential(hb, bnd), args.steps, args.warmup,
                                                         flags=0)[0], 4)
            schedules[f"overlap_{n}"] = round(run(plans.overlap(hb, bnd), args.steps, args.warmup, flags=0)[0], 4)
        if stack:
            # cross-layer pipelining of the same plans
            for n in (2, 4):
                ov = plans.overlap(hb, plans.even_bounds(T, n))
                schedules[f"overlap_{n}_pipelined"] = round(run(ov, args.steps, args.warmup,
                                                                flags=abi.NF_STACK_PIPELINE)[0], 4)
        log("schedules (ms/step): " + ", ".join(f"{k} {v:.3f}" for k, v in schedules.items()))

    # a stack's decode-attention launch is its layer's launch on the same batch
    traffic = counted_traffic(wl.extra.get("layer_workload", wl.name), args.seed, launches_per_step / n_layers)
    tokens_per_s = T / (ms * 1e-3)
    step_gemm_flops = alg["gemm_flops"] * n_layers
    mfma_frac = step_gemm_flops / (ms * 1e-3) / PEAK_BF16
    t_lb = n_layers * max(alg["gemm_flops"] / PEAK_BF16, alg["layer_bytes"] / PEAK_HBM)

    kv_io = None
    if args.kv_io and not stack:
        def one_step():
            abi.nf_layer_forward(ctx, cfg, w_descs[0], xd.data_ptr(), yd.data_ptr(), hb, p_descs[0], plan, stream)
        one_step.pool_desc = p_descs[0]
        kv_io = kv_io_probe(abi, torch, ctx, cfg, shape, b, one_step, stream, steps=args.steps)
        log(f"kv io: {kv_io}")

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        def fetch_blocks(layer, ids):
            idx = torch.from_numpy(np.asarray(ids, dtype=np.int64)).cuda()
            kp = k16s[layer].index_select(0, idx).cpu().numpy().view(np.uint16)
            vp = v16s[layer].index_select(0, idx).cpu().numpy().view(np.uint16)
            return kp, vp

        if w is None:  # device-drawn weights: the oracle reads host copies of the layers it runs
            n_cpu = max(1, min(args.cpu_layers, n_layers))
            ws_host = [wds[l].host_bits() for l in range(n_cpu)]
        else:
            ws_host = [w]
        cpu = cpu_baseline(shape, b, ws_host, x, args.seed, args.cpu_decode_sample, fetch_blocks, n_layers)
        log(f"cpu oracle: {cpu['value']} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "n_layers": n_layers,
            "stack_pipelined": (not args.no_pipeline) if stack else None,
            "dense_batch": T,
            "n_decode": b.n_decode,
            "prefill_len": b.prefill_len.tolist(),
            "decode_ctx_range": list(wl.decode_ctx_range),
            "seed": args.seed,
            "plan": plan_desc,
            "decode_grid": args.decode_grid,
            "decode_split": args.decode_split,
            "prefill_chunk": args.prefill_chunk,
            "decode_nbuf": args.decode_nbuf,
            "decode_ring": args.decode_ring,
            "gemm_variant": args.gemm_variant,
            "gemm_variants": args.gemm_variants or None,
        },
        "step_ms_distribution": dict(dist, steps=args.steps),
        "mfma_frac_of_bf16_peak": round(mfma_frac, 4),
        # against the fastest of this run's own GEMM kernels (the profiled-peak convention)
        "own_gemm_peak_tflops": own_peak,
        "mfma_frac_of_own_gemm_peak": None if not own_peak else round(step_gemm_flops / (ms * 1e-3) / 1e12 / own_peak, 4),
        "hbm_copy_gbps": round(copy_gbps, 1),
        "decode_attn_vs_copy": round(achieved / 1e9 / copy_gbps, 4),
        "layer_gemm_tflops": round(step_gemm_flops / (ms * 1e-3) / 1e12, 1),
        "layer_roofline_frac": round(t_lb / (ms * 1e-3), 4),
        "sequential_ms_per_step": None if seq_ms is None else round(seq_ms, 4),
        "speedup_vs_sequential": None if seq_ms is None else round(seq_ms / ms, 4),
        "schedules_ms_per_step": schedules,
        "roofline": {
            "kernel": "decode_attn_kernel<128> (paged GQA decode attention, split-KV)",
            "bound": "hbm",
            "achieved": round(achieved / 1e9, 1),
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM, 4),
            "traffic": traffic,
            "traffic_unit": "bytes/launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a known-size copy)",
            "traffic_vs_algorithmic": None if traffic is None else round(traffic / bytes_per_launch, 4),
            "bytes_per_launch": int(bytes_per_launch),
            "avg_launch_ms": round(dec_avg_ms, 4),
            "launches_per_step": launches_per_step,
        },
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in breakdown.items()},
        "cpu_baseline": cpu,
        "kv_io": kv_io,
    }
    if args.vendor_gemm and not shape.n_experts:
        out["gemm_vs_vendor"] = gemm_vs_vendor(ctx, shape, T, args.seed)
    abi.nf_ctx_destroy(ctx)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
