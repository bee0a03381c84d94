"""The profiler's tables: the committed ones the search reads (CPU), and a fresh profile of
the tiny layer written by nf_profile_ops and nf_profile_interference (GPU)."""

import glob
import json
import os

import pytest

from synth import workloads as sw
from tests.profile_schema import check_dbest, check_interference

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLES = os.path.join(ROOT, "nano_intra_overlap_amd", "tables")


def _workload_of(path, suffix):
    return os.path.basename(path)[: -len(suffix)]


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(TABLES, "*_dbest.json"))))
def test_committed_dbest_tables(path):
    from nano_intra_overlap_amd import abi

    wl = sw.WORKLOADS[_workload_of(path, "_dbest.json")]
    with open(path) as f:
        d = json.load(f)
    assert d["cfg"]["hidden"] == wl.shape.hidden and d["cfg"]["ffn"] == wl.shape.ffn
    check_dbest(d, wl.n_tokens, n_variants=len(abi.nf_gemm_variants()))


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(TABLES, "*_interference.json"))))
def test_committed_interference_tables(path):
    wl = sw.WORKLOADS[_workload_of(path, "_interference.json")]
    with open(path) as f:
        r = json.load(f)
    assert r["cfg"]["hidden"] == wl.shape.hidden
    check_interference(r, r_grid=[0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875])
    assert 0 <= r["min_gain"] < 1


@pytest.mark.gpu
def test_profilers_on_the_tiny_layer(tmp_path):
    """Both profilers on the tiny shape at 128-token steps up to its batch size rounded up
    to 256: the files they write have the tables' schema and sane values."""
    torch = pytest.importorskip("torch")
    from nano_intra_overlap_amd import abi
    from tests.gpu_util import log_case

    wl = sw.WORKLOADS["tiny"]
    b = sw.make_batch("tiny", 0)
    hb = abi.HostBatch.from_batch(b)
    cfg = abi.make_cfg(wl.shape)
    ctx = abi.nf_ctx_create(0)
    try:
        d_path, r_path = str(tmp_path / "dbest.json"), str(tmp_path / "rp.json")
        log_case("nf_profile_ops on the tiny layer")
        abi.nf_profile_ops(ctx, cfg, hb, b.num_blocks, 128, 256, d_path)
        log_case("nf_profile_interference on the tiny layer")
        abi.nf_profile_interference(ctx, cfg, hb, b.num_blocks, [0.25, 0.5], r_path)
        torch.cuda.synchronize()
    finally:
        abi.nf_ctx_destroy(ctx)
    with open(d_path) as f:
        # the tiny shape's products take a few microseconds, launch latency included: their
        # times need not grow with the batch
        check_dbest(json.load(f), 256, n_variants=len(abi.nf_gemm_variants()), monotone=False)
    with open(r_path) as f:
        r = json.load(f)
    r["min_gain"] = 0.0
    check_interference(r, r_grid=[0.25, 0.5])
    # the search takes both files
    json.loads(abi.nf_plan_search(d_path, r_path, hb, max_nano=2, granularity=128))
