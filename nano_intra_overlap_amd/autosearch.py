"""Offline auto-search for one workload: profile, then two-stage search.

1. nf_profile_ops          -> D_best table (every nano-op kind x batch size, best variant)
2. nf_profile_interference -> interference table (P of the GEMM and decode-attention
                              nano-ops for each resource split)
3. nf_plan_search          -> plan JSON for nf_layer_forward (an overlapped plan only when
                              predicted faster than the sequential one by more than the
                              table's min_gain, --min-gain)

Run on the GPU machine: ``python -m nano_intra_overlap_amd.autosearch --workload llama3_8b_layer``.
Tables land in nano_intra_overlap_amd/tables/<workload>_{dbest,interference,plan}.json.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
TABLES = os.path.join(PKG, "tables")


def table_paths(workload: str, seed: int = 0):
    base = os.path.join(TABLES, f"{workload}")
    return base + "_dbest.json", base + "_interference.json", base + f"_plan_seed{seed}.json"


def search_plan(workload: str, seed: int = 0, max_nano: int = 4, granularity: int = 128, dbest=None, rp=None):
    """Run the (host-only) two-stage search for a workload's seeded batch; returns the JSON text."""
    sys.path.insert(0, os.path.dirname(PKG))
    from synth import workloads as sw

    from . import abi

    # a layer stack uses the tables profiled for its layer shape
    d, r, _ = table_paths(sw.WORKLOADS[workload].extra.get("layer_workload", workload))
    b = sw.make_batch(workload, seed)
    return abi.nf_plan_search(dbest or d, rp or r, abi.HostBatch.from_batch(b), max_nano=max_nano,
                              granularity=granularity)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama3_8b_layer")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--step", type=int, default=128)
    ap.add_argument("--max-nano", type=int, default=4)
    ap.add_argument("--r-grid", default="0.125,0.25,0.375,0.5,0.625,0.75,0.875",
                    help="memory-stream CU shares to profile (each with the compute op on the complement mask "
                         "and on the whole GPU)")
    ap.add_argument("--skip-profile", action="store_true")
    ap.add_argument("--skip-ops", action="store_true", help="keep the D_best table, profile interference only")
    ap.add_argument("--min-gain", type=float, default=0.06,
                    help="an overlapped plan must be predicted this fraction faster than the sequential one "
                         "(written into the interference table; measured on MI355X: overlapped plans run 6-10%% "
                         "slower than predicted, the sequential plan 3-9%%)")
    args = ap.parse_args()

    sys.path.insert(0, os.path.dirname(PKG))
    from synth import workloads as sw

    from . import abi

    os.makedirs(TABLES, exist_ok=True)
    wl = sw.WORKLOADS[args.workload]
    b = sw.make_batch(args.workload, args.seed)
    hb = abi.HostBatch.from_batch(b)
    cfg = abi.make_cfg(wl.shape)
    d, r, p = table_paths(args.workload, args.seed)
    if not args.skip_profile:
        ctx = abi.nf_ctx_create(0)
        t0 = time.time()
        if not args.skip_ops:
            abi.nf_profile_ops(ctx, cfg, hb, b.num_blocks, args.step, wl.n_tokens, d)
            print(f"[autosearch] D_best table -> {d} ({time.time() - t0:.1f} s)", flush=True)
        t0 = time.time()
        grid = [float(x) for x in args.r_grid.split(",") if x]
        abi.nf_profile_interference(ctx, cfg, hb, b.num_blocks, grid, r)
        print(f"[autosearch] interference table -> {r} ({time.time() - t0:.1f} s)", flush=True)
        abi.nf_ctx_destroy(ctx)
    if os.path.exists(r):
        with open(r) as f:
            table = json.load(f)
        table["min_gain"] = args.min_gain
        with open(r, "w") as f:
            json.dump(table, f, indent=1)
            f.write("\n")
    text = search_plan(args.workload, args.seed, args.max_nano, args.step)
    with open(p, "w") as f:
        f.write(text + "\n")
    rec = json.loads(text)
    print(f"[autosearch] plan -> {p}: {rec['summary']}; sequential predicted {rec['sequential_ms']:.3f} ms",
          flush=True)


if __name__ == "__main__":
    main()
