"""Two-stage pipeline search: the library's nf_plan_search against hand-computed schedules,
the pages' Stage I rules, and a brute-force Python search over the same space."""

import json
import os

import numpy as np
import pytest

from oracle import schedule as osch
from synth import workloads as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_values.json")))


@pytest.fixture(scope="module")
def abi():
    from nano_intra_overlap_amd import abi as a

    a.load()
    return a


def _write(tmp_path, name, obj):
    p = tmp_path / name
    p.write_text(json.dumps(obj))
    return str(p)


def _table(rng, scale=1.0):
    """A synthetic D_best table: dense ops ~linear in tokens with a fixed cost (weight
    loads), decode attention linear in decode tokens, prefill quadratic-ish."""
    sizes = list(range(128, 2049, 128))
    a, b = rng.uniform(0.02, 0.08), rng.uniform(1e-4, 5e-4)
    return {
        "KQV": [[s, scale * (a + b * s)] for s in sizes],
        "O": [[s, scale * (0.6 * a + 0.7 * b * s)] for s in sizes],
        "UGD": [[s, scale * (3 * a + 4 * b * s)] for s in sizes],
        "DECATTN": [[s, scale * rng.uniform(5e-4, 1.2e-3) * s] for s in sizes],
        "PFATTN": [[s, scale * 2e-8 * s * s + 0.01] for s in sizes],
    }


# ------------------------------------------------------------------------ simulator pins


def test_simulator_hand_computed_two_nano_schedule():
    # 2 decode-only nano-batches; compute: KQV0 KQV1 O0 U0 O1 U1; memory: D0 D1
    b = sw.batch_from_lengths(np.full(4, 10), [], seed=0)
    bounds = [0, 2, 4]
    deps = {}
    for x, y in osch.dependencies(b, bounds):
        deps.setdefault(y, set()).add(x)
    K, D, P, O, U = osch.KQV, osch.DECATTN, osch.PFATTN, osch.O, osch.UGD
    dur = {(K, 0): 1, (K, 1): 1, (D, 0): 5, (D, 1): 5, (P, 0): 0, (P, 1): 0, (O, 0): 1, (O, 1): 1,
           (U, 0): 2, (U, 1): 2}
    st = osch.structure(2, 2, True)
    # KQV0 [0,1] KQV1 [1,2]; D0 [1,6]; D1 [6,11]; O0 [6,7] U0 [7,9]; O1 [11,12] U1 [12,14]
    assert osch.simulate(st, deps, dur) == 14
    # Stage II: with both streams at half speed while overlapping, T = D_best / P
    speeds = dict(p_gemm_both=0.5, p_mem_both=0.5, p_gemm_alone=1.0, p_mem_alone=1.0)
    only_two = {k: 0 for k in dur}
    only_two[(K, 0)] = 0
    only_two[(D, 0)] = 4
    only_two[(O, 0)] = 0
    only_two[(U, 0)] = 0
    only_two[(K, 1)] = 4
    # D0 and KQV1 both run from t=0 at half speed: each takes 4 / 0.5 = 8
    assert osch.simulate(st, deps, only_two, speeds) == pytest.approx(8.0)


def test_stage1_rules_from_the_pages():
    rules = GOLDEN["stage1_rules"]
    for n in (2, 3, 4):
        for bounds in osch.all_bounds(2048, n, rules["granularity"]):
            sizes = np.diff(bounds)
            assert (sizes % rules["granularity"] == 0).all() and (sizes >= rules["min_batch"]).all()
            assert sum(sizes) == 2048
    # the page's example splits are among the enumerated ones
    ex = GOLDEN["nano_batch_examples"]
    two = [0, ex["up_two"][0][1], 2048]
    four = [0] + [r[1] for r in ex["kqv_four"]]
    assert two in list(osch.all_bounds(2048, 2, 128))
    assert four in list(osch.all_bounds(2048, 4, 128))


# ------------------------------------------------------------------------ library vs oracle


def _batch(rng, T=1024):
    p = int(rng.integers(100, 400))
    return sw.batch_from_lengths(rng.integers(200, 2000, T - p), [p], seed=1)


@pytest.mark.parametrize("seed", range(4))
def test_search_matches_brute_force(abi, tmp_path, seed):
    rng = np.random.default_rng(seed)
    b = _batch(rng)
    table = _table(rng)
    configs = [
        {"name": "shared", "p_gemm_both": 0.7, "p_mem_both": 0.8},
        {"name": "mem25", "r_mem": 0.25, "p_gemm_both": 0.85, "p_mem_both": 0.5, "p_gemm_alone": 0.75,
         "p_mem_alone": 0.55},
        # per compute kind: short products starve beside the memory op (as measured on a shared
        # GPU), the FFN product does not
        {"name": "shared_kinds", "p_gemm_both": 0.9, "p_mem_both": 0.85,
         "p_gemm_both_kind": {"KQV": 0.12, "O": 0.2, "UGD": 0.9}, "p_gemm_alone_kind": {"KQV": 0.95},
         "p_mem_both_kind": {"KQV": 0.95, "UGD": 0.7}},
    ]
    dpath = _write(tmp_path, "dbest.json", {"ops": table})
    rpath = _write(tmp_path, "rp.json", {"configs": configs})
    hb = abi.HostBatch.from_batch(b)
    plan = json.loads(abi.nf_plan_search(dpath, rpath, hb, max_nano=4, granularity=128))
    speeds = [{**{k: c.get(k, 1.0) for k in ("p_gemm_both", "p_mem_both", "p_gemm_alone", "p_mem_alone")},
               **{k: c[k] for k in ("p_gemm_both_kind", "p_gemm_alone_kind", "p_mem_both_kind") if k in c}}
              for c in configs]
    best, stage1 = osch.search(b, table, speeds, max_nano=4, gran=128, top_k=8)
    assert plan["stage1"]["best_ms"] == pytest.approx(stage1, rel=1e-9)
    assert plan["predicted_ms"] == pytest.approx(best, rel=1e-6)
    # the plan is valid for the executor
    from nano_intra_overlap_amd import plans

    hp, rec = plans.from_json(json.dumps(plan))
    abi.nf_plan_dependencies(hb, hp)


def test_search_per_kind_compute_interference(abi, tmp_path):
    """A table that gives the compute speed beside the memory op per compute kind: the
    library and the brute-force search agree, and the per-kind speeds change the outcome
    against the same table without them (so the kinds are actually read)."""
    rng = np.random.default_rng(21)
    b = _batch(rng)
    table = _table(rng)
    plain = {"name": "shared", "p_gemm_both": 0.9, "p_mem_both": 0.9}
    kinds = dict(plain, p_gemm_both_kind={"KQV": 0.3, "O": 0.45, "UGD": 0.95}, p_gemm_alone_kind={"O": 0.98},
                 p_mem_both_kind={"KQV": 0.97, "O": 0.93, "UGD": 0.6})
    dpath = _write(tmp_path, "dbest.json", {"ops": table})
    hb = abi.HostBatch.from_batch(b)
    got = {}
    for name, cfg in (("plain", plain), ("kinds", kinds)):
        rpath = _write(tmp_path, f"rp_{name}.json", {"configs": [cfg]})
        plan = json.loads(abi.nf_plan_search(dpath, rpath, hb, max_nano=4, granularity=128))
        speeds = {k: cfg.get(k, 1.0) for k in ("p_gemm_both", "p_mem_both", "p_gemm_alone", "p_mem_alone")}
        speeds.update({k: cfg[k] for k in ("p_gemm_both_kind", "p_gemm_alone_kind", "p_mem_both_kind") if k in cfg})
        best, _ = osch.search(b, table, [speeds], max_nano=4, gran=128, top_k=8)
        assert plan["predicted_ms"] == pytest.approx(best, rel=1e-6), name
        got[name] = plan["predicted_ms"]
    assert got["kinds"] > got["plain"]


def _masks(r):
    per = round(32 * r)
    mem = [0] * 8
    gem = [0] * 8
    for i in range(256):
        (mem if i // 8 >= 32 - per else gem)[i // 32] |= 1 << (i % 32)
    return gem, mem


def _per_kind_table(r, kqv_full, o_full, ugd_full, masked_kqv=0.95, masked_ugd=0.6):
    """A masked entry and its unmasked-compute partner at memory share r."""
    gem, mem = _masks(r)
    masked = {"name": f"mask_r{r}", "r_mem": r, "p_gemm_both": masked_ugd, "p_mem_both": 0.55,
              "p_gemm_alone": 0.7, "p_mem_alone": 0.85,
              "p_gemm_both_kind": {"KQV": masked_kqv, "O": 0.6, "UGD": masked_ugd},
              "p_gemm_alone_kind": {"KQV": 1.0, "O": 0.65, "UGD": 0.7},
              "p_mem_both_kind": {"KQV": 0.75, "O": 0.6, "UGD": 0.45}, "cu_masks": [gem, mem]}
    full = {"name": f"mask_r{r}_gemm_full", "r_mem": r, "gemm_full": True, "p_gemm_both": ugd_full,
            "p_mem_both": 0.35, "p_gemm_alone": 1.0, "p_mem_alone": 0.85,
            "p_gemm_both_kind": {"KQV": kqv_full, "O": o_full, "UGD": ugd_full},
            "p_gemm_alone_kind": {"KQV": 1.0, "O": 1.0, "UGD": 1.0},
            "p_mem_both_kind": {"KQV": 0.3, "O": 0.33, "UGD": 0.6}, "cu_masks": [[0xFFFFFFFF] * 8, mem]}
    return [masked, full]


def _speeds(c):
    out = {k: c.get(k, 1.0) for k in ("p_gemm_both", "p_mem_both", "p_gemm_alone", "p_mem_alone")}
    out.update({k: c[k] for k in ("p_gemm_both_kind", "p_gemm_alone_kind", "p_mem_both_kind", "r_mem",
                                   "gemm_full", "cu_masks") if k in c})
    return out


@pytest.mark.parametrize("seed", range(3))
def test_search_per_kind_resource_share(abi, tmp_path, seed):
    """Stage II gives each compute kind its own share: the complement of the memory mask or
    the whole GPU beside it. The library and the brute-force search agree on the best
    makespan; a table where KQV keeps its speed on the complement mask but the FFN product
    needs the whole GPU yields a three-stream plan with the compute ops on one lane."""
    rng = np.random.default_rng(40 + seed)
    b = _batch(rng)
    table = _table(rng)
    configs = _per_kind_table(0.375, kqv_full=0.3, o_full=0.5, ugd_full=0.95, masked_kqv=1.0, masked_ugd=0.5) + \
        _per_kind_table(0.25, kqv_full=0.35, o_full=0.4, ugd_full=0.9, masked_kqv=0.95, masked_ugd=0.55)
    dpath = _write(tmp_path, "dbest.json", {"ops": table})
    rpath = _write(tmp_path, "rp.json", {"configs": configs})
    hb = abi.HostBatch.from_batch(b)
    plan = json.loads(abi.nf_plan_search(dpath, rpath, hb, max_nano=4, granularity=128))
    best, _ = osch.search(b, table, [_speeds(c) for c in configs], max_nano=4, gran=128, top_k=8)
    assert plan["predicted_ms"] == pytest.approx(best, rel=1e-6)
    # the same tables without the partner entries: never better
    only_masked = [c for c in configs if not c.get("gemm_full")]
    best_masked, _ = osch.search(b, table, [_speeds(c) for c in only_masked], max_nano=4, gran=128, top_k=8)
    assert best <= best_masked + 1e-12
    assert plan["n_streams"] == 3 and plan["unmasked_kinds"] and len(plan["cu_masks"]) == 3
    lanes = {(o["kind"], o["nano"]): (o["stream"], o["lane"]) for o in plan["ops"]}
    compute = [v for (k, _), v in lanes.items() if k in (osch.KQV, osch.O, osch.UGD)]
    assert {ln for _, ln in compute} == {0} and {st for st, _ in compute} == {0, 2}
    for (k, _), (st, ln) in lanes.items():
        full = osch.KIND_NAMES[k] in plan["unmasked_kinds"]
        if k in (osch.KQV, osch.O, osch.UGD):
            assert st == (2 if full else 0)
    from nano_intra_overlap_amd import plans

    hp, _ = plans.from_json(json.dumps(plan))
    edges, order = abi.nf_plan_dependencies(hb, hp)
    # the compute lane runs one op at a time: consecutive lane ops on different streams
    # are joined by an edge
    listed = [(o["kind"], o["nano"], o["stream"], o["lane"]) for o in plan["ops"]]
    lane0 = [i for i, o in enumerate(listed) if o[3] == 0]
    for a, c in zip(lane0, lane0[1:]):
        if listed[a][2] != listed[c][2]:
            assert (a, c) in edges


def test_lane_edges_in_plan_graph(abi):
    """op_lane: consecutive ops of one lane on different streams get an ordering edge; on
    the same stream they need none; without lanes nothing is added; a lane out of range is
    refused."""
    b = sw.batch_from_lengths(np.full(256, 300), [], seed=0)
    hb = abi.HostBatch.from_batch(b)
    K, D, P, O, U = osch.KQV, osch.DECATTN, osch.PFATTN, osch.O, osch.UGD
    bounds = [0, 128, 256]
    ops = [(K, 0, 0), (D, 0, 1), (P, 0, 1), (K, 1, 2), (D, 1, 1), (P, 1, 1), (O, 0, 0), (U, 0, 2),
           (O, 1, 0), (U, 1, 0)]
    lanes = [0, 1, 1, 0, 1, 1, 0, 0, 0, 0]
    plain, _ = abi.nf_plan_dependencies(hb, abi.HostPlan(bounds, ops, 3))
    laned, order = abi.nf_plan_dependencies(hb, abi.HostPlan(bounds, ops, 3, lanes=lanes))
    added = set(laned) - set(plain)
    # lane 0 in listed order: 0(s0) 3(s2) 6(s0) 7(s2) 8(s0) 9(s0)
    assert added == {(0, 3), (3, 6), (6, 7), (7, 8)} - set(plain)
    assert set(plain) <= set(laned)
    pos = {op: i for i, op in enumerate(order)}
    for i, j in laned:
        assert pos[i] < pos[j]
    with pytest.raises(abi.NanoflowError):
        abi.nf_plan_dependencies(hb, abi.HostPlan(bounds, ops, 3, lanes=[0] * 9 + [3]))


@pytest.mark.parametrize("min_gain", [0.0, 0.05, 0.3])
def test_search_min_gain(abi, tmp_path, min_gain):
    """The table's min_gain: an overlapped plan is taken only when predicted faster than the
    sequential one by more than that fraction (brute force applies the same rule)."""
    rng = np.random.default_rng(33)
    b = _batch(rng)
    table = _table(rng)
    cfg = {"name": "shared", "p_gemm_both": 0.8, "p_mem_both": 0.85}
    dpath = _write(tmp_path, "dbest.json", {"ops": table})
    rpath = _write(tmp_path, "rp.json", {"configs": [cfg], "min_gain": min_gain})
    plan = json.loads(abi.nf_plan_search(dpath, rpath, abi.HostBatch.from_batch(b), max_nano=4, granularity=128))
    speeds = {k: cfg.get(k, 1.0) for k in ("p_gemm_both", "p_mem_both", "p_gemm_alone", "p_mem_alone")}
    best, _ = osch.search(b, table, [speeds], max_nano=4, gran=128, top_k=8, min_gain=min_gain)
    assert plan["predicted_ms"] == pytest.approx(best, rel=1e-6)
    overlapped = plan["n_streams"] >= 2
    assert overlapped == (best < plan["sequential_ms"] * (1 - min_gain))
    if overlapped:
        assert plan["predicted_ms"] < plan["sequential_ms"] * (1 - min_gain)
    else:
        assert plan["predicted_ms"] == pytest.approx(plan["sequential_ms"])
    if min_gain == 0.3:
        assert not overlapped
    rpath = _write(tmp_path, "rp_bad.json", {"configs": [cfg], "min_gain": 1.5})
    with pytest.raises(abi.NanoflowError):
        abi.nf_plan_search(dpath, rpath, abi.HostBatch.from_batch(b), max_nano=4, granularity=128)


def test_search_prefers_sequential_when_interference_is_ruinous(abi, tmp_path):
    rng = np.random.default_rng(9)
    b = _batch(rng)
    table = _table(rng)
    dpath = _write(tmp_path, "dbest.json", {"ops": table})
    rpath = _write(tmp_path, "rp.json", {"configs": [{"name": "bad", "p_gemm_both": 0.2, "p_mem_both": 0.2}]})
    plan = json.loads(abi.nf_plan_search(dpath, rpath, abi.HostBatch.from_batch(b), max_nano=4, granularity=128))
    assert plan["n_streams"] == 1 and plan["bounds"] == [0, b.n_tokens]
    assert plan["predicted_ms"] == pytest.approx(plan["sequential_ms"])


def test_search_without_interference_table_overlaps(abi, tmp_path):
    rng = np.random.default_rng(3)
    b = _batch(rng)
    dpath = _write(tmp_path, "dbest.json", {"ops": _table(rng)})
    plan = json.loads(abi.nf_plan_search(dpath, "", abi.HostBatch.from_batch(b), max_nano=4, granularity=128))
    assert plan["n_streams"] == 2 and len(plan["bounds"]) >= 3
    assert plan["predicted_ms"] < plan["sequential_ms"]


def test_search_rejects_bad_inputs(abi, tmp_path):
    b = _batch(np.random.default_rng(0))
    hb = abi.HostBatch.from_batch(b)
    with pytest.raises(abi.NanoflowError) as e:
        abi.nf_plan_search(str(tmp_path / "missing.json"), "", hb)
    assert e.value.status == abi.NF_E_IO
    bad = _write(tmp_path, "bad.json", {"ops": {"KQV": [[128, 0.1]]}})
    with pytest.raises(abi.NanoflowError):
        abi.nf_plan_search(bad, "", hb)
    with pytest.raises(abi.NanoflowError):
        abi.nf_plan_search(_write(tmp_path, "d.json", {"ops": _table(np.random.default_rng(1))}), "", hb, max_nano=0)
