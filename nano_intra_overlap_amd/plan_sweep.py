"""Time overlap plans with per-kind resource shares against the sequential layer.

The two-stage search predicts from profiled tables; this tool measures. For one workload's
seeded batch it times, with the layer's own kernels on the GPU:

* the sequential layer (one nano-batch on the caller's stream);
* nano-batching without overlap (``plans.sequential``) and the overlap template on a
  shared GPU (``plans.overlap``) for 2 and 3 even nano-batches;
* the overlap template with the memory stream on a CU mask of ``m`` CUs per XCD and every
  subset of the dense kinds (KQV, O, Up/Gate/Down) on an unmasked third stream, the rest on
  the complement mask — the per-operation shares of the NanoFlow summary page ("Auto-Search
  Stage II: Refining the Pipeline"), one compute lane across the two compute streams.

For a layer stack (``--workload llama3_8b_32layer``, optionally ``--layers n`` of its layers)
every plan runs through the stack call with cross-layer pipelining, whose steady state
overlaps each nano-batch's decode attention with the other nano-batch's whole dense half
(its O, Up/Gate/Down and the next layer's KQV); ``--no-pipeline`` issues layer by layer.

Each plan: 5 warm-up steps, then the faster of two runs of 20 steps. Run on the GPU machine:
``python -m nano_intra_overlap_amd.plan_sweep --workload llama2_70b_tp8_layer``.
"""

from __future__ import annotations

import argparse
import itertools
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama3_8b_layer")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--mem-cus", default="4,8,12,16,20,24", help="memory-stream CUs per XCD (of 32) to try")
    ap.add_argument("--nano", default="2,3", help="even nano-batch counts to try")
    ap.add_argument("--kinds", default="all",
                    help="'all': every subset of dense kinds on the unmasked stream; 'none': all masked")
    ap.add_argument("--layers", type=int, default=0, help="layer stacks: time the first n layers (0 = all)")
    ap.add_argument("--no-pipeline", action="store_true", help="layer stacks: issue layer by layer")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--grids", default="", help="shared-GPU overlap: decode-attention workgroup caps to try")
    ap.add_argument("--bounds", default="",
                    help="extra nano-batch bounds to try (';'-separated lists, e.g. '0,768,2048')")
    ap.add_argument("--o-on-memory", action="store_true",
                    help="shared-GPU overlap: also try O issued on the memory stream after its attention")
    ap.add_argument("--ov-variants", default="",
                    help="GEMM tile variants (KQV, O, Up/Gate, Down; -1 = library choice) for the overlapped "
                         "plans; several sets separated by ';'")
    args = ap.parse_args()

    sys.path.insert(0, os.path.dirname(PKG))
    import numpy as np
    import torch

    from synth import workloads as sw
    from synth.workloads import make_kv_pool_torch

    from . import abi, plans
    from .device import DevicePool, DeviceWeights, bf16_tensor

    wl = sw.WORKLOADS[args.workload]
    shape = wl.shape
    b = sw.make_batch(args.workload, args.seed)
    T = b.n_tokens
    n_layers = shape.n_layers if args.layers <= 0 else min(args.layers, shape.n_layers)
    stack = shape.n_layers > 1
    print(f"{args.workload}: T={T} decode={b.n_decode} prefill={b.prefill_len.tolist()} layers={n_layers}",
          flush=True)
    if stack:  # per-layer weights from the counter generator and pools, drawn on the device
        wds = [DeviceWeights.from_int16(sw.make_weights_counter_torch(shape, args.seed, l, device="cuda"))
               for l in range(n_layers)]
        pools = [DevicePool.from_int16(*make_kv_pool_torch(shape, b.num_blocks, args.seed, layer=l, device="cuda"))
                 for l in range(n_layers)]
    else:
        wds = [DeviceWeights(sw.make_weights(shape, args.seed), "cuda")]
        pools = [DevicePool.from_int16(*make_kv_pool_torch(shape, b.num_blocks, args.seed, device="cuda"))]
    xd = bf16_tensor(sw.make_x(shape, T, args.seed), "cuda")
    yd = torch.empty_like(xd)
    bt_dev = torch.from_numpy(np.ascontiguousarray(b.block_table)).cuda()
    hb = abi.HostBatch.from_batch(b, block_table_dev_ptr=bt_dev.data_ptr())
    cfg = abi.make_cfg(shape)
    ctx = abi.nf_ctx_create(0)
    stream = torch.cuda.current_stream().cuda_stream

    flags = 0 if args.no_pipeline else abi.NF_STACK_PIPELINE
    w_descs, p_descs = [w.desc for w in wds], [p.desc for p in pools]

    def step(plan):
        if stack:
            abi.nf_stack_forward(ctx, cfg, w_descs, xd.data_ptr(), yd.data_ptr(), hb, p_descs, plan,
                                 flags if plan is not None else 0, stream)
        else:
            abi.nf_layer_forward(ctx, cfg, w_descs[0], xd.data_ptr(), yd.data_ptr(), hb, p_descs[0], plan, stream)

    def time_plan(plan, steps=args.steps, warmup=5):
        for _ in range(warmup):
            step(plan)
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                step(plan)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / steps)
        return best

    rows = []

    def run(name, plan):
        ms = time_plan(plan)
        rows.append((ms, name))
        print(f"{name:56s} {ms:.4f} ms", flush=True)

    kind_slots = ((abi.NF_OP_KQV, 0), (abi.NF_OP_O, 0), (abi.NF_OP_UGD, 0), (abi.NF_OP_UGD, 1))
    run("sequential (one nano-batch)", None)
    letter = {abi.NF_OP_KQV: "K", abi.NF_OP_O: "O", abi.NF_OP_UGD: "U"}
    bsets = [plans.even_bounds(T, int(x)) for x in args.nano.split(",") if x]
    bsets += [[int(v) for v in x.split(",")] for x in args.bounds.split(";") if x]
    for bnd in bsets:
        n = f"{len(bnd) - 1}" + ("" if bnd == plans.even_bounds(T, len(bnd) - 1) else f" {bnd}")
        run(f"{n} nano: nano-batching only", plans.sequential(hb, bnd))
        run(f"{n} nano: overlap, shared GPU", plans.overlap(hb, bnd))
        for vset in (args.ov_variants.split(";") if args.ov_variants else [""]):
            vs = [int(x) for x in vset.split(",")] if vset else [-1] * 4
            for (kind, which), v in zip(kind_slots, vs):
                abi.nf_ctx_set_gemm_variant(ctx, kind, which, v)
            tagv = f", variants {vset}" if vset else ""
            for grid in (int(x) for x in args.grids.split(",") if x):
                p = plans.overlap(hb, bnd)
                run(f"{n} nano: overlap, shared GPU, attention grid {grid}{tagv}",
                    abi.HostPlan(bnd, p.ops, p.n_streams, None, grid))
                if args.o_on_memory:
                    p = plans.overlap(hb, bnd, memory_kinds=(abi.NF_OP_O,))
                    run(f"{n} nano: overlap, O on memory stream, attention grid {grid}{tagv}",
                        abi.HostPlan(bnd, p.ops, p.n_streams, None, grid))
            for kind, which in kind_slots:
                abi.nf_ctx_set_gemm_variant(ctx, kind, which, -1)
        for per in (int(x) for x in args.mem_cus.split(",") if x):
            cm = abi.cu_mask(per_xcd=32 - per, offset=0)
            mm = abi.cu_mask(per_xcd=per, offset=32 - per)
            for k in (range(4) if args.kinds == "all" else (0,)):
                for kinds in itertools.combinations((abi.NF_OP_KQV, abi.NF_OP_O, abi.NF_OP_UGD), k):
                    tag = "".join(letter[x] for x in kinds) or "-"
                    run(f"{n} nano: memory {per}/32 CUs, unmasked [{tag}]",
                        plans.overlap(hb, bnd, cm, mm, unmasked_kinds=kinds))
    seq = rows[0][0]
    print("\nfastest:", flush=True)
    for ms, name in sorted(rows)[:8]:
        print(f"  {ms:.4f} ms  {ms / seq:6.3f}x  {name}", flush=True)
    abi.nf_ctx_destroy(ctx)


if __name__ == "__main__":
    main()
