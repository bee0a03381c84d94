// Two-stage pipeline search (NanoFlow summary page, "Auto-Search Stage I: Pipeline
// Structure Search" and "Auto-Search Stage II: Refining the Pipeline"; slides "Auto-Search
// Stage 1" and "Stage 2").
//
// Stage I fixes the structure assuming no interference: the number of nano-batches n, their
// sizes (multiples of the granularity, summing to the dense batch; at least the granularity
// each), and the order of nano-operations on each stream (ops of one class never overlap:
// one stream per class, compute = KQV/O/UGD, memory = decode attention, prefill attention on
// either). Each nano-op takes its interference-free best time D_best(kind, size) from the
// profile; dependencies follow range intersection. The makespan of the list schedule (an op
// starts when its stream is free and its producers are done) is minimised by exhaustive
// enumeration of the same discrete space an MILP would search (every split, lookahead and
// prefill placement), preferring fewer nano-batches on ties (fewer weight reloads).
//
// Stage II keeps the structure and chooses the resource split between the two streams from
// the measured interference table: for each configuration c, an op runs at P_both(c) of its
// best speed while an op of the other class runs and at P_alone(c) otherwise (a masked
// stream is slower even alone). The schedule is re-simulated with these rates (time advances
// from one completion to the next) and the configuration with the shortest makespan wins.
// The compute rate, and the memory op's rate beside it, may be given per compute kind (KQV,
// O, UGD measured each against the memory op): on a shared GPU a short product beside
// decode attention waits for CU slots far longer than the long FFN product does.
// Resource share per compute kind: the memory class keeps one CU mask (share R, over the
// table's grid), and each compute kind (KQV, O, UGD) takes either the complement of that
// mask or the whole GPU beside it (the table's "gemm_full" entry of the same R), so the
// kinds can hold different shares (the pages' per-operation R). Mixed choices need three
// streams (masked compute, memory, unmasked compute); the compute ops stay one lane that
// runs one op at a time in the listed order.
// Extension: the K best Stage-I structures and the single-stream sequential plan are all
// re-ranked under interference, since on this GPU interference can reverse Stage I's order;
// an overlapped plan is taken only when predicted faster than the sequential one by more
// than the table's "min_gain" fraction (0 when absent).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <sstream>

#include "nf_batch.h"
#include "nf_json.h"

namespace nf {
namespace {

struct Curve {
  std::vector<std::pair<double, double>> pts;  // (size, ms), sorted
  double at(double x) const {
    if (x <= 0 || pts.empty()) return 0.0;
    if (x <= pts.front().first) return pts.front().second * x / pts.front().first;
    for (size_t i = 1; i < pts.size(); ++i)
      if (x <= pts[i].first) {
        const double x0 = pts[i - 1].first, x1 = pts[i].first, y0 = pts[i - 1].second, y1 = pts[i].second;
        return y0 + (y1 - y0) * (x - x0) / (x1 - x0);
      }
    if (pts.size() == 1) return pts[0].second * x / pts[0].first;
    const auto& a = pts[pts.size() - 2];
    const auto& b = pts.back();
    return b.second + (b.second - a.second) * (x - b.first) / (b.first - a.first);
  }
};

struct Profile {
  Curve op[NF_OP_KINDS];
};

struct InterfCfg {
  std::string name;
  double r = -1.0;  // memory stream CU share (-1: shared GPU, no masks)
  double pg_both = 1, pm_both = 1, pg_alone = 1, pm_alone = 1;
  // per compute kind (KQV, O, UGD) when the table measured each against the memory op;
  // otherwise pg_both / pg_alone. pm_both_k: the memory op's speed beside each compute kind.
  double pg_both_k[NF_OP_KINDS] = {1, 1, 1, 1, 1}, pg_alone_k[NF_OP_KINDS] = {1, 1, 1, 1, 1};
  double pm_both_k[NF_OP_KINDS] = {1, 1, 1, 1, 1};
  bool has_masks = false;
  bool gemm_full = false;  // compute op unmasked beside a masked memory op
  uint32_t masks[2][NF_CU_MASK_WORDS];
  int decode_grid = 0;
};

// Stage II's placement of compute kinds: kinds in full_kinds run as in `full` (unmasked
// beside the memory mask), the others on the complement mask of the configuration.
struct Placement {
  const InterfCfg* full = nullptr;
  unsigned full_kinds = 0;  // bit k: kind k on the unmasked stream
};

const int kComputeKinds[3] = {NF_OP_KQV, NF_OP_O, NF_OP_UGD};

unsigned placement_kinds(unsigned choice) {  // bit i of choice: kComputeKinds[i] unmasked
  unsigned m = 0;
  for (int i = 0; i < 3; ++i)
    if (choice >> i & 1u) m |= 1u << kComputeKinds[i];
  return m;
}

const char* kKindNames[NF_OP_KINDS] = {"KQV", "DECATTN", "PFATTN", "O", "UGD"};

bool load_profile(const char* path, Profile& P, std::string& err) {
  json::Value v;
  if (!json::parse_file(path, v, err)) return false;
  const json::Value& ops = v.at("ops");
  if (!ops.is_obj()) {
    err = "D_best table lacks an 'ops' object";
    return false;
  }
  for (int k = 0; k < NF_OP_KINDS; ++k) {
    const json::Value& a = ops.at(kKindNames[k]);
    if (!a.is_arr()) continue;
    for (auto& e : a.arr) {
      if (e.is_arr() && e.arr.size() >= 2 && e.arr[0].is_num() && e.arr[1].is_num())
        P.op[k].pts.push_back({e.arr[0].num, e.arr[1].num});
      else if (e.is_obj() && e.has("size") && e.has("ms"))
        P.op[k].pts.push_back({e.number("size", 0), e.number("ms", 0)});
    }
    std::sort(P.op[k].pts.begin(), P.op[k].pts.end());
  }
  for (int k : {NF_OP_KQV, NF_OP_O, NF_OP_UGD})
    if (P.op[k].pts.empty()) {
      err = std::string("D_best table has no entries for ") + kKindNames[k];
      return false;
    }
  return true;
}

bool load_interference(const char* path, std::vector<InterfCfg>& out, double& min_gain, std::string& err) {
  out.clear();
  min_gain = 0.0;
  if (!path || !*path) {
    InterfCfg c;
    c.name = "ideal";
    out.push_back(c);
    return true;
  }
  json::Value v;
  if (!json::parse_file(path, v, err)) return false;
  min_gain = v.number("min_gain", 0.0);
  if (!(min_gain >= 0.0 && min_gain < 1.0)) {
    err = "interference table: min_gain must lie in [0, 1)";
    return false;
  }
  const json::Value& cs = v.at("configs");
  if (!cs.is_arr() || cs.arr.empty()) {
    err = "interference table lacks a non-empty 'configs' array";
    return false;
  }
  for (auto& e : cs.arr) {
    InterfCfg c;
    c.name = e.at("name").kind == json::Value::Str ? e.at("name").str : "cfg";
    c.r = e.number("r_mem", -1.0);
    c.pg_both = e.number("p_gemm_both", 1.0);
    c.pm_both = e.number("p_mem_both", 1.0);
    c.pg_alone = e.number("p_gemm_alone", 1.0);
    c.pm_alone = e.number("p_mem_alone", 1.0);
    for (int k = 0; k < NF_OP_KINDS; ++k) {
      c.pg_both_k[k] = c.pg_both;
      c.pg_alone_k[k] = c.pg_alone;
      c.pm_both_k[k] = c.pm_both;
    }
    for (int k : {(int)NF_OP_KQV, (int)NF_OP_O, (int)NF_OP_UGD}) {
      c.pg_both_k[k] = e.at("p_gemm_both_kind").number(kKindNames[k], c.pg_both);
      c.pg_alone_k[k] = e.at("p_gemm_alone_kind").number(kKindNames[k], c.pg_alone);
      c.pm_both_k[k] = e.at("p_mem_both_kind").number(kKindNames[k], c.pm_both);
      if (!(c.pg_both_k[k] > 0 && c.pg_alone_k[k] > 0 && c.pm_both_k[k] > 0)) {
        err = "interference entry '" + c.name + "' has a non-positive speed";
        return false;
      }
    }
    c.decode_grid = (int)e.number("decode_grid", 0.0);
    c.gemm_full = e.at("gemm_full").kind == json::Value::Bool && e.at("gemm_full").b;
    const json::Value& m = e.at("cu_masks");
    if (m.is_arr() && m.arr.size() == 2) {
      c.has_masks = true;
      for (int s = 0; s < 2; ++s)
        for (int w = 0; w < NF_CU_MASK_WORDS; ++w)
          c.masks[s][w] = (uint32_t)(m.arr[s].is_arr() && (int)m.arr[s].arr.size() > w ? m.arr[s].arr[w].num : 0);
    }
    if (!(c.pg_both > 0 && c.pm_both > 0 && c.pg_alone > 0 && c.pm_alone > 0)) {
      err = "interference entry '" + c.name + "' has a non-positive speed";
      return false;
    }
    out.push_back(c);
  }
  return true;
}

// A candidate structure: nano-batch bounds and per-stream op orders.
struct Structure {
  std::vector<int32_t> bounds;
  int lookahead = 1;
  bool pf_on_memory = true;
  bool sequential = false;
  std::vector<std::vector<std::pair<int, int>>> streams;  // (kind, nano) per stream, in order
};

struct SimResult {
  bool ok = false;
  double makespan = 0;
  std::vector<double> start, end;  // per op index (kind * n + nano)
};

// Durations of every nano-op (interference-free best times).
std::vector<double> op_durations(const BatchLayout& L, const PlanGraph& g, const Profile& P) {
  const int n = g.n_nano;
  std::vector<double> d(NF_OP_KINDS * n, 0.0);
  for (auto& op : g.ops) {
    double t = 0.0;
    const int rows = g.bounds[op.nano + 1] - g.bounds[op.nano];
    switch (op.kind) {
      case NF_OP_KQV:
      case NF_OP_O:
      case NF_OP_UGD: t = P.op[op.kind].at(rows); break;
      case NF_OP_DECATTN: t = P.op[NF_OP_DECATTN].at(op.r1 - op.r0); break;
      case NF_OP_PFATTN:
        for (int32_t r : op.prefill_reqs) t += P.op[NF_OP_PFATTN].at(L.req[r].t1 - L.req[r].t0);
        break;
    }
    d[op.kind * n + op.nano] = t;
  }
  return d;
}

// Event-driven simulation of two (or one) in-order streams with dependency waits. The rate
// of a running op depends on whether an op of the other stream runs at the same time.
SimResult simulate(const Structure& S, const PlanGraph& g, const std::vector<double>& dur, const InterfCfg& c,
                   const Placement* pl = nullptr) {
  const int n = g.n_nano;
  const int n_ops = NF_OP_KINDS * n;
  SimResult R;
  R.start.assign(n_ops, -1.0);
  R.end.assign(n_ops, -1.0);
  // dependency lists by (kind, nano) index
  std::vector<std::vector<int>> deps(n_ops);
  for (size_t i = 0; i < g.ops.size(); ++i) {
    const int a = g.ops[i].kind * n + g.ops[i].nano;
    for (int32_t d : g.deps[i]) deps[a].push_back(g.ops[d].kind * n + g.ops[d].nano);
  }
  const int ns = (int)S.streams.size();
  std::vector<size_t> pos(ns, 0);
  std::vector<int> cur(ns, -1);
  std::vector<double> remaining(ns, 0.0);
  double t = 0.0;
  int done = 0;
  const bool compute_is_stream0 = true;
  for (int guard = 0; guard < 4 * n_ops + 8; ++guard) {
    // start every stream whose head op is ready; zero-length ops complete at once and may
    // unblock another stream's head, so repeat until nothing changes
    for (bool progress = true; progress;) {
      progress = false;
      for (int s = 0; s < ns; ++s) {
        while (cur[s] < 0 && pos[s] < S.streams[s].size()) {
        const auto ko = S.streams[s][pos[s]];
        const int id = ko.first * n + ko.second;
        bool ready = true;
        for (int d : deps[id])
          if (R.end[d] < 0 || R.end[d] > t + 1e-12) ready = false;
        if (!ready) break;
        progress = true;
        if (dur[id] <= 0.0) {  // empty op: completes at once
          R.start[id] = R.end[id] = t;
          ++done;
          ++pos[s];
          continue;
        }
        cur[s] = id;
        remaining[s] = dur[id];
        R.start[id] = t;
        ++pos[s];
        }
      }
    }
    int active = 0;
    for (int s = 0; s < ns; ++s) active += cur[s] >= 0;
    if (active == 0) {
      bool all = true;
      for (int s = 0; s < ns; ++s) all &= pos[s] == S.streams[s].size();
      if (all) break;
      return R;  // deadlock: a head op waits for an op that can never run
    }
    // rates; a compute op placed on the unmasked stream takes the "full" entry's speeds, and
    // so does the memory op beside it
    auto cfg_of = [&](int id) -> const InterfCfg& {
      return (pl && pl->full && (pl->full_kinds >> (id / n) & 1u)) ? *pl->full : c;
    };
    std::vector<double> rate(ns, 1.0);
    for (int s = 0; s < ns; ++s) {
      if (cur[s] < 0) continue;
      const bool is_compute = (s == 0) == compute_is_stream0;
      const bool other = active > 1;
      if (ns == 1) {
        rate[s] = 1.0;
      } else if (is_compute) {
        const InterfCfg& cc = cfg_of(cur[s]);
        rate[s] = other ? cc.pg_both_k[cur[s] / n] : cc.pg_alone_k[cur[s] / n];
      } else {
        const int g_op = cur[compute_is_stream0 ? 0 : 1];
        rate[s] = other ? cfg_of(g_op).pm_both_k[g_op / n] : c.pm_alone;
      }
    }
    // next completion
    double dt = 1e300;
    for (int s = 0; s < ns; ++s)
      if (cur[s] >= 0) dt = std::min(dt, remaining[s] / rate[s]);
    t += dt;
    for (int s = 0; s < ns; ++s) {
      if (cur[s] < 0) continue;
      remaining[s] -= dt * rate[s];
      if (remaining[s] <= 1e-12 * std::max(1.0, dur[cur[s]])) {
        R.end[cur[s]] = t;
        ++done;
        cur[s] = -1;
      }
    }
  }
  if (done != n_ops) return R;
  R.ok = true;
  R.makespan = 0;
  for (double e : R.end) R.makespan = std::max(R.makespan, e);
  return R;
}

Structure make_structure(const std::vector<int32_t>& bounds, int a, bool pf_mem) {
  Structure S;
  S.bounds = bounds;
  S.lookahead = a;
  S.pf_on_memory = pf_mem;
  const int n = (int)bounds.size() - 1;
  S.streams.assign(2, {});
  auto& cs = S.streams[0];
  auto& ms = S.streams[1];
  for (int j = 0; j < std::min(a, n); ++j) cs.push_back({NF_OP_KQV, j});
  for (int j = 0; j < n; ++j) {
    if (!pf_mem) cs.push_back({NF_OP_PFATTN, j});
    cs.push_back({NF_OP_O, j});
    cs.push_back({NF_OP_UGD, j});
    if (j + a < n) cs.push_back({NF_OP_KQV, j + a});
    ms.push_back({NF_OP_DECATTN, j});
    if (pf_mem) ms.push_back({NF_OP_PFATTN, j});
  }
  return S;
}

Structure make_sequential(int32_t T) {
  Structure S;
  S.bounds = {0, T};
  S.sequential = true;
  S.streams.assign(1, {});
  for (int k = 0; k < NF_OP_KINDS; ++k) S.streams[0].push_back({k, 0});
  return S;
}

// Enumerate bounds: cuts at multiples of gran strictly inside (0, T).
void for_each_bounds(int32_t T, int n, int gran, const std::function<void(const std::vector<int32_t>&)>& fn) {
  std::vector<int32_t> cuts;
  for (int32_t c = gran; c < T; c += gran) cuts.push_back(c);
  if (n == 1) {
    fn({0, T});
    return;
  }
  if ((int)cuts.size() < n - 1) return;
  std::vector<int> idx(n - 1);
  for (int i = 0; i < n - 1; ++i) idx[i] = i;
  while (true) {
    std::vector<int32_t> b = {0};
    for (int i : idx) b.push_back(cuts[i]);
    b.push_back(T);
    fn(b);
    int i = n - 2;
    while (i >= 0 && idx[i] == (int)cuts.size() - (n - 1) + i) --i;
    if (i < 0) break;
    ++idx[i];
    for (int j = i + 1; j < n - 1; ++j) idx[j] = idx[j - 1] + 1;
  }
}

struct Candidate {
  Structure S;
  double stage1 = 0;
};

}  // namespace
}  // namespace nf

using namespace nf;

static void put(char* dst, size_t cap, const std::string& s) {
  if (!dst || cap == 0) return;
  const size_t n = std::min(cap - 1, s.size());
  memcpy(dst, s.data(), n);
  dst[n] = 0;
}

extern "C" nf_status nf_plan_search(const char* dbest_json, const char* rp_json, const nf_batch_desc* batch,
                                    int32_t max_nano, int32_t granularity, char* plan_json_out, size_t cap) {
  if (!dbest_json || !batch || max_nano < 1 || max_nano > 8 || granularity < 1 || !plan_json_out || cap < 64) {
    put(plan_json_out, cap, "nf_plan_search: bad argument");
    return NF_E_ARG;
  }
  std::string err;
  Profile P;
  if (!load_profile(dbest_json, P, err)) {
    put(plan_json_out, cap, err);
    return NF_E_IO;
  }
  std::vector<InterfCfg> cfgs;
  double min_gain = 0.0;
  if (!load_interference(rp_json, cfgs, min_gain, err)) {
    put(plan_json_out, cap, err);
    return NF_E_IO;
  }
  // token layout of the batch (lengths only; the search needs no pool)
  BatchLayout L;
  int64_t t = 0;
  for (int32_t r = 0; r < batch->n_decode + batch->n_prefill; ++r) {
    ReqInfo ri;
    ri.decode = r < batch->n_decode;
    const int32_t q = ri.decode ? 1 : batch->prefill_len[r - batch->n_decode];
    if (q < 1) {
      put(plan_json_out, cap, "prefill length < 1");
      return NF_E_ARG;
    }
    ri.t0 = (int32_t)t;
    ri.t1 = (int32_t)(t + q);
    ri.cached = 0;
    ri.n_keys = q;
    L.req.push_back(ri);
    t += q;
  }
  L.T = (int32_t)t;
  if (L.T < 1) {
    put(plan_json_out, cap, "empty batch");
    return NF_E_ARG;
  }

  auto graph_for = [&](const std::vector<int32_t>& bounds, PlanGraph& g) -> bool {
    const int n = (int)bounds.size() - 1;
    std::vector<int32_t> k, j, s;
    for (int kk = 0; kk < NF_OP_KINDS; ++kk)
      for (int jj = 0; jj < n; ++jj) {
        k.push_back(kk);
        j.push_back(jj);
        s.push_back(0);
      }
    nf_plan p{n, bounds.data(), 1, nullptr, (int32_t)k.size(), k.data(), j.data(), s.data()};
    std::string e;
    return build_plan_graph(L, &p, g, e) == NF_OK;
  };

  // ---- Stage I ---------------------------------------------------------------------------
  InterfCfg ideal;
  ideal.name = "ideal";
  std::vector<Candidate> cands;
  int64_t evaluated = 0;
  for (int n = 1; n <= max_nano; ++n) {
    for_each_bounds(L.T, n, granularity, [&](const std::vector<int32_t>& bounds) {
      PlanGraph g;
      if (!graph_for(bounds, g)) return;
      const std::vector<double> dur = op_durations(L, g, P);
      for (int a = 1; a <= n; ++a)
        for (int pfm = 0; pfm < 2; ++pfm) {
          Structure S = make_structure(bounds, a, pfm == 1);
          SimResult r = simulate(S, g, dur, ideal);
          ++evaluated;
          if (!r.ok) continue;
          cands.push_back({S, r.makespan});
        }
    });
  }
  if (cands.empty()) {
    put(plan_json_out, cap, "no feasible structure");
    return NF_E_PLAN;
  }
  std::stable_sort(cands.begin(), cands.end(), [](const Candidate& x, const Candidate& y) {
    const double tol = 1e-9 * std::max(1.0, std::max(x.stage1, y.stage1));
    if (std::fabs(x.stage1 - y.stage1) > tol) return x.stage1 < y.stage1;
    return x.S.bounds.size() < y.S.bounds.size();  // fewer nano-batches on ties
  });
  const Candidate best1 = cands.front();

  // ---- Stage II ---------------------------------------------------------------------------
  const size_t K = std::min<size_t>(8, cands.size());
  std::vector<Candidate> pool(cands.begin(), cands.begin() + K);
  Candidate seq{make_sequential(L.T), 0};
  {
    PlanGraph g;
    graph_for(seq.S.bounds, g);
    seq.stage1 = simulate(seq.S, g, op_durations(L, g, P), ideal).makespan;
  }
  pool.push_back(seq);
  // the unmasked-compute partner of a masked entry: the "gemm_full" entry of the same R
  auto partner = [&](size_t k) -> const InterfCfg* {
    if (!cfgs[k].has_masks || cfgs[k].gemm_full) return nullptr;
    for (auto& f : cfgs)
      if (f.gemm_full && f.has_masks && std::fabs(f.r - cfgs[k].r) < 1e-6) return &f;
    return nullptr;
  };
  double best_ms = 1e300;
  int best_c = -1, best_k = -1;
  unsigned best_choice = 0;  // bit i: kComputeKinds[i] on the unmasked stream
  std::vector<double> best_start;
  for (size_t ci = 0; ci < pool.size(); ++ci) {
    PlanGraph g;
    graph_for(pool[ci].S.bounds, g);
    const std::vector<double> dur = op_durations(L, g, P);
    for (size_t k = 0; k < cfgs.size(); ++k) {
      if (pool[ci].S.sequential && k > 0) break;  // one stream: no interference, full GPU
      // every kind on the complement mask (choice 0); with a partner entry also the mixed
      // choices (all kinds unmasked is the partner entry itself)
      const InterfCfg* full = pool[ci].S.sequential ? nullptr : partner(k);
      for (unsigned choice = 0; choice < (full ? 7u : 1u); ++choice) {
        const Placement pl{full, placement_kinds(choice)};
        SimResult r = simulate(pool[ci].S, g, dur, pool[ci].S.sequential ? ideal : cfgs[k], &pl);
        if (!r.ok) continue;
        if (r.makespan < best_ms - 1e-12) {
          best_ms = r.makespan;
          best_c = (int)ci;
          best_k = pool[ci].S.sequential ? -1 : (int)k;
          best_choice = choice;
          best_start = r.start;
        }
      }
    }
  }
  // an overlapped plan has to beat the sequential one by more than the table's min_gain
  // (the interference model's observed error on this device); otherwise sequential
  {
    const int seq_c = (int)pool.size() - 1;
    if (best_c != seq_c && best_ms > seq.stage1 * (1.0 - min_gain)) {
      PlanGraph g;
      graph_for(seq.S.bounds, g);
      SimResult r = simulate(seq.S, g, op_durations(L, g, P), ideal);
      best_ms = r.makespan;
      best_c = seq_c;
      best_k = -1;
      best_choice = 0;
      best_start = r.start;
    }
  }
  const Candidate& win = pool[best_c];
  const int n = (int)win.S.bounds.size() - 1;
  // listing: ops ordered by simulated start time (ties: stream 0 first, then stream order)
  struct Item {
    double t;
    int s, p, kind, nano;
  };
  std::vector<Item> items;
  for (int s = 0; s < (int)win.S.streams.size(); ++s)
    for (int p = 0; p < (int)win.S.streams[s].size(); ++p) {
      const auto ko = win.S.streams[s][p];
      items.push_back({best_start[ko.first * n + ko.second], s, p, ko.first, ko.second});
    }
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
    if (a.t != b.t) return a.t < b.t;
    if (a.s != b.s) return a.s < b.s;
    return a.p < b.p;
  });
  // streams: lane 0 (compute) and lane 1 (memory) as in the structure; a mixed placement
  // adds stream 2, unmasked, for the compute kinds placed there (still lane 0)
  const unsigned full_kinds = placement_kinds(best_choice);
  const bool mixed = best_choice != 0;
  auto stream_of = [&](const Item& it) {
    return (mixed && it.s == 0 && (full_kinds >> it.kind & 1u)) ? 2 : it.s;
  };
  std::ostringstream o;
  o << "{\"bounds\": [";
  for (size_t i = 0; i < win.S.bounds.size(); ++i) o << (i ? ", " : "") << win.S.bounds[i];
  o << "], \"n_streams\": " << win.S.streams.size() + (mixed ? 1 : 0) << ", \"ops\": [";
  for (size_t i = 0; i < items.size(); ++i)
    o << (i ? ", " : "") << "{\"kind\": " << items[i].kind << ", \"nano\": " << items[i].nano
      << ", \"stream\": " << stream_of(items[i]) << ", \"lane\": " << items[i].s << "}";
  o << "], \"cu_masks\": ";
  if (best_k >= 0 && cfgs[best_k].has_masks) {
    o << "[";
    for (int s = 0; s < 2; ++s) {
      o << (s ? ", " : "") << "[";
      for (int w = 0; w < NF_CU_MASK_WORDS; ++w) o << (w ? ", " : "") << cfgs[best_k].masks[s][w];
      o << "]";
    }
    if (mixed) {
      o << ", [";
      for (int w = 0; w < NF_CU_MASK_WORDS; ++w) o << (w ? ", " : "") << 0xFFFFFFFFu;
      o << "]";
    }
    o << "]";
  } else {
    o << "null";
  }
  std::string cfg_name = best_k >= 0 ? cfgs[best_k].name : "sequential";
  if (mixed) {
    cfg_name += " + unmasked";
    for (int i = 0; i < 3; ++i)
      if (best_choice >> i & 1u) cfg_name += std::string(" ") + kKindNames[kComputeKinds[i]];
  }
  o << ", \"decode_grid\": " << (best_k >= 0 ? cfgs[best_k].decode_grid : 0);
  o << ", \"interference_config\": " << json::quote(cfg_name);
  o << ", \"r_mem\": " << json::num(best_k >= 0 ? cfgs[best_k].r : -1.0);
  o << ", \"unmasked_kinds\": [";
  for (int i = 0, first = 1; i < 3; ++i)
    if (best_choice >> i & 1u) {
      o << (first ? "" : ", ") << json::quote(kKindNames[kComputeKinds[i]]);
      first = 0;
    }
  o << "]";
  o << ", \"predicted_ms\": " << json::num(best_ms);
  o << ", \"sequential_ms\": " << json::num(seq.stage1);
  o << ", \"lookahead\": " << win.S.lookahead << ", \"prefill_on_memory_stream\": "
    << (win.S.pf_on_memory ? "true" : "false");
  o << ", \"stage1\": {\"evaluated\": " << evaluated << ", \"best_ms\": " << json::num(best1.stage1)
    << ", \"best_bounds\": [";
  for (size_t i = 0; i < best1.S.bounds.size(); ++i) o << (i ? ", " : "") << best1.S.bounds[i];
  o << "], \"best_lookahead\": " << best1.S.lookahead << "}";
  std::ostringstream sm;
  sm << (win.S.sequential ? "sequential" : "overlap") << ", " << n << " nano-batch(es), predicted "
     << json::num(best_ms) << " ms (" << (best_k >= 0 ? cfg_name : std::string("one stream")) << ")";
  o << ", \"summary\": " << json::quote(sm.str()) << "}";
  const std::string out = o.str();
  if (out.size() + 1 > cap) {
    put(plan_json_out, cap, "plan does not fit the output buffer");
    return NF_E_CAPACITY;
  }
  put(plan_json_out, cap, out);
  return NF_OK;
}
