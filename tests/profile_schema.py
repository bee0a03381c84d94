"""Checks of the profiler's output files: the D_best table (best interference-free time of
every nano-operation kind at every batch size) and the pairwise interference table (P of a
GEMM nano-op and of decode attention under each resource split), as the pages describe them
(summary page, "Kernel Profiling and Interference Modeling"). Shared by the CPU test of the
committed tables and the GPU test of a fresh profile."""

from __future__ import annotations

import math

KINDS = ("KQV", "DECATTN", "PFATTN", "O", "UGD")
DENSE = ("KQV", "O", "UGD")
# P is a speed relative to the warmed best of the same kernel alone; timing noise can put an
# undisturbed run a few percent above that best
P_MAX = 1.05
# D_best of a dense product may dip by timing noise from one size to the next
MONOTONE_SLACK = 0.02


def check_dbest(d: dict, max_tokens: int, n_variants: int | None = None, monotone: bool = True):
    step = d["step"]
    assert step > 0 and step % 128 == 0, step
    assert d["cu"] > 0
    assert set(d["ops"]) == set(KINDS), sorted(d["ops"])
    sizes = list(range(step, max_tokens + 1, step))
    for kind, rows in d["ops"].items():
        assert [int(r[0]) for r in rows] == sizes, (kind, [r[0] for r in rows])
        times = [float(r[1]) for r in rows]
        assert all(math.isfinite(t) and t > 0 for t in times), (kind, times)
        if kind in DENSE and monotone:
            for a, b in zip(times, times[1:]):
                assert b >= a * (1 - MONOTONE_SLACK), (kind, a, b)
        if kind == "DECATTN":  # [tokens, ms, split-KV blocks, blocks per step, ring]
            for r in rows:
                assert int(r[2]) >= 0 and int(r[3]) in (1, 2) and 2 <= int(r[4]) <= 4, r
    for kind, rows in d["best_variants"].items():
        assert kind in DENSE, kind
        assert [int(r[0]) for r in rows] == sizes, kind
        if n_variants is not None:
            assert all(0 <= int(r[1]) < n_variants for r in rows), (kind, rows)


def check_interference(r: dict, r_grid=None):
    assert r["device_cus"] > 0
    assert r["t_gemm_best_ms"] > 0 and r["t_mem_best_ms"] > 0
    names = [c["name"] for c in r["configs"]]
    assert "shared" in names, names
    masked = [c for c in r["configs"] if c["name"].startswith("mask_r") and not c.get("gemm_full")]
    full = [c for c in r["configs"] if c.get("gemm_full")]
    if r_grid is not None:
        assert sorted(round(c["r_mem"], 6) for c in masked) == sorted(round(x, 6) for x in r_grid)
    # a table with unmasked-compute entries has one per masked entry, same memory mask
    if full:
        assert sorted(round(c["r_mem"], 6) for c in full) == sorted(round(c["r_mem"], 6) for c in masked)
        by_r = {round(c["r_mem"], 6): c for c in masked}
        for c in full:
            assert c["cu_masks"][1] == by_r[round(c["r_mem"], 6)]["cu_masks"][1], c["name"]
            assert all(w == 0xFFFFFFFF for w in c["cu_masks"][0]), c["name"]
    for c in r["configs"]:
        ps = [c["p_gemm_both"], c["p_mem_both"], c["p_gemm_alone"], c["p_mem_alone"]]
        for key in ("p_gemm_both_kind", "p_mem_both_kind", "p_gemm_alone_kind"):
            assert set(c[key]) == set(DENSE), (c["name"], key)
            ps += list(c[key].values())
        assert all(0 < p <= P_MAX for p in ps), (c["name"], ps)
        if c["name"].startswith("mask_r"):
            assert 0 < c["r_mem"] < 1
            assert c["cu_masks"] is not None and len(c["cu_masks"]) == 2
            # the two streams' CU masks are disjoint (the compute one is the whole GPU in a
            # "gemm_full" entry) and leave no XCD without CUs
            g, m = c["cu_masks"]
            if not c.get("gemm_full"):
                assert all((a & b) == 0 for a, b in zip(g, m)), c["name"]
            for mask in (g, m):
                per = [0] * 8
                for i in range(32 * len(mask)):
                    if mask[i // 32] >> (i % 32) & 1:
                        per[i % 8] += 1
                assert min(per) > 0 and min(per) == max(per), (c["name"], per)
        else:
            assert c["r_mem"] == -1
