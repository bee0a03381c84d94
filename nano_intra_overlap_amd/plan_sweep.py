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
    if shape.n_layers != 1:
        raise SystemExit("plan_sweep times single-layer workloads")
    b = sw.make_batch(args.workload, args.seed)
    T = b.n_tokens
    print(f"{args.workload}: T={T} decode={b.n_decode} prefill={b.prefill_len.tolist()}", flush=True)
    wd = DeviceWeights(sw.make_weights(shape, args.seed), "cuda")
    xd = bf16_tensor(sw.make_x(shape, T, args.seed), "cuda")
    yd = torch.empty_like(xd)
    k16, v16 = make_kv_pool_torch(shape, b.num_blocks, args.seed, device="cuda")
    pool = DevicePool.from_int16(k16, v16)
    bt_dev = torch.from_numpy(np.ascontiguousarray(b.block_table)).cuda()
    hb = abi.HostBatch.from_batch(b, block_table_dev_ptr=bt_dev.data_ptr())
    cfg = abi.make_cfg(shape)
    ctx = abi.nf_ctx_create(0)
    stream = torch.cuda.current_stream().cuda_stream

    def step(plan):
        abi.nf_layer_forward(ctx, cfg, wd.desc, xd.data_ptr(), yd.data_ptr(), hb, pool.desc, plan, stream)

    def time_plan(plan, steps=20, warmup=5):
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

    run("sequential (one nano-batch)", None)
    letter = {abi.NF_OP_KQV: "K", abi.NF_OP_O: "O", abi.NF_OP_UGD: "U"}
    for n in (int(x) for x in args.nano.split(",") if x):
        bnd = plans.even_bounds(T, n)
        run(f"{n} nano: nano-batching only", plans.sequential(hb, bnd))
        run(f"{n} nano: overlap, shared GPU", plans.overlap(hb, bnd))
        for per in (int(x) for x in args.mem_cus.split(",") if x):
            cm = abi.cu_mask(per_xcd=32 - per, offset=0)
            mm = abi.cu_mask(per_xcd=per, offset=32 - per)
            for k in range(4):
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
