// Host-side batch layout and nano-operation DAG (pure C++, no GPU).
//
// Batch layout: decode requests first (one token each), then prefill chunks (slides,
// "Batch Formation"). Token t of request r sits at position cached_r + (t - t0_r) and its
// K/V go to slot table[r][pos / 16] * 16 + pos % 16 ("Inside nano-vLLM": slot mapping;
// "LLM Inference Performance": PagedAttention block table).
//
// Dependencies: nano-operation B depends on A iff their parent operations are dependent
// and their token ranges intersect (NanoFlow summary page, "Auto-Search Stage I",
// constraints on dependencies). Parent graph of the layer: KQV -> decode attention,
// KQV -> prefill attention, both attentions -> O, O -> UGD. A prefill attention nano-op
// owns the chunks whose last token lies in its nano-batch, and its range is the union of
// those chunks' rows, so it waits for every KQV nano-op that produced part of them.
#include "nf_batch.h"

#include <algorithm>
#include <cstdio>
#include <cstring>

namespace nf {

static std::string fmt(const char* f, long a = 0, long b = 0, long c = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

nf_status check_cfg(const nf_layer_cfg& c, std::string& err) {
  if (c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 || c.ffn <= 0) {
    err = "layer shape has a non-positive size";
    return NF_E_ARG;
  }
  if (c.block_size != 16) {
    err = fmt("block_size %ld unsupported (16 only)", c.block_size);
    return NF_E_UNSUPPORTED;
  }
  if (c.head_dim != 64 && c.head_dim != 128) {
    err = fmt("head_dim %ld unsupported (64 or 128)", c.head_dim);
    return NF_E_UNSUPPORTED;
  }
  if (c.n_q_heads % c.n_kv_heads != 0 || c.n_q_heads / c.n_kv_heads > 16) {
    err = fmt("n_q_heads %ld / n_kv_heads %ld must be an integer <= 16", c.n_q_heads, c.n_kv_heads);
    return NF_E_UNSUPPORTED;
  }
  if (c.hidden % 8 || c.ffn % 8) {
    err = "hidden and ffn must be multiples of 8";
    return NF_E_UNSUPPORTED;
  }
  if (!(c.rms_eps >= 0.0f) || !(c.rope_base > 0.0f)) {
    err = "rms_eps must be >= 0 and rope_base > 0";
    return NF_E_ARG;
  }
  if (c.n_experts < 0) {
    err = "n_experts must be >= 0";
    return NF_E_ARG;
  }
  if (c.n_experts > 0) {
    if (!moe_experts_supported(c.n_experts) || c.top_k != 2) {
      err = fmt("MoE with %ld experts, top %ld unsupported (4, 8 or 16 experts, top 2)", c.n_experts, c.top_k);
      return NF_E_UNSUPPORTED;
    }
    if (c.hidden % 32 || c.ffn % 32) {
      err = "MoE layers need hidden and ffn multiples of 32";
      return NF_E_UNSUPPORTED;
    }
  }
  return NF_OK;
}

nf_status build_layout(const nf_layer_cfg& cfg, const nf_batch_desc& b, int32_t num_blocks, BatchLayout& L,
                       std::string& err) {
  const int32_t BS = cfg.block_size;
  if (b.n_decode < 0 || b.n_prefill < 0) {
    err = "negative request count";
    return NF_E_ARG;
  }
  if ((b.n_decode > 0 && !b.decode_ctx_len) || (b.n_prefill > 0 && !b.prefill_len)) {
    err = "null length array";
    return NF_E_ARG;
  }
  const int32_t n_req = b.n_decode + b.n_prefill;
  if (n_req > 0 && (!b.block_table || b.max_blocks <= 0)) {
    err = "null block table or max_blocks <= 0";
    return NF_E_ARG;
  }
  if (num_blocks <= 0) {
    err = "pool holds no blocks";
    return NF_E_ARG;
  }
  L.req.clear();
  L.req.reserve(n_req);
  int64_t t = 0;
  for (int32_t r = 0; r < n_req; ++r) {
    ReqInfo ri;
    ri.decode = r < b.n_decode;
    int64_t cached, qlen;
    if (ri.decode) {
      cached = b.decode_ctx_len[r];
      qlen = 1;
      if (cached < 0) {
        err = fmt("decode request %ld: context length %ld < 0", r, (long)cached);
        return NF_E_ARG;
      }
    } else {
      const int32_t j = r - b.n_decode;
      qlen = b.prefill_len[j];
      cached = b.prefill_prefix_len ? b.prefill_prefix_len[j] : 0;
      if (qlen < 1 || cached < 0) {
        err = fmt("prefill chunk %ld: length %ld / prefix %ld invalid", j, (long)qlen, (long)cached);
        return NF_E_ARG;
      }
    }
    const int64_t n_keys = cached + qlen;
    const int64_t need = (n_keys + BS - 1) / BS;
    if (need > b.max_blocks) {
      err = fmt("request %ld needs %ld blocks but its table row holds %ld", r, (long)need, b.max_blocks);
      return NF_E_BLOCK_TABLE_SHORT;
    }
    const int32_t* row = b.block_table + (size_t)r * b.max_blocks;
    for (int64_t i = 0; i < need; ++i) {
      if (row[i] < 0 || row[i] >= num_blocks) {
        err = fmt("request %ld: logical block %ld maps to %ld, outside the pool", r, (long)i, row[i]);
        return NF_E_BLOCK_RANGE;
      }
    }
    if (t + qlen > INT32_MAX / 2 || n_keys > INT32_MAX / 2) {
      err = "batch too large";
      return NF_E_CAPACITY;
    }
    ri.t0 = (int32_t)t;
    ri.t1 = (int32_t)(t + qlen);
    ri.cached = (int32_t)cached;
    ri.n_keys = (int32_t)n_keys;
    L.req.push_back(ri);
    t += qlen;
  }
  L.T = (int32_t)t;
  L.pos.resize(L.T);
  L.slot.resize(L.T);
  for (int32_t r = 0; r < n_req; ++r) {
    const ReqInfo& ri = L.req[r];
    const int32_t* row = b.block_table + (size_t)r * b.max_blocks;
    for (int32_t tt = ri.t0; tt < ri.t1; ++tt) {
      const int32_t p = ri.cached + (tt - ri.t0);
      L.pos[tt] = p;
      L.slot[tt] = row[p / BS] * BS + p % BS;
    }
  }
  // every new token must own a distinct slot
  std::vector<int32_t> s(L.slot);
  std::sort(s.begin(), s.end());
  for (size_t i = 1; i < s.size(); ++i) {
    if (s[i] == s[i - 1]) {
      err = fmt("two new tokens write KV slot %ld (block %ld)", s[i], s[i] / BS);
      return NF_E_SLOT_ALIAS;
    }
  }
  return NF_OK;
}

bool parent_depends(int32_t a, int32_t b) {
  switch (b) {
    case NF_OP_DECATTN:
    case NF_OP_PFATTN: return a == NF_OP_KQV;
    case NF_OP_O: return a == NF_OP_DECATTN || a == NF_OP_PFATTN;
    case NF_OP_UGD: return a == NF_OP_O;
    default: return false;
  }
}

static bool intersects(const NanoOp& a, const NanoOp& b) {
  for (auto& x : a.rows)
    for (auto& y : b.rows)
      if (std::max(x.first, y.first) < std::min(x.second, y.second)) return true;
  return false;
}

nf_status build_plan_graph(const BatchLayout& L, const nf_plan* plan, PlanGraph& g, std::string& err) {
  g = PlanGraph();
  const int32_t T = L.T;
  std::vector<int32_t> kinds, nanos, streams, lanes;
  if (!plan) {
    g.n_nano = 1;
    g.n_streams = 1;
    g.bounds = {0, T};
    for (int32_t k = 0; k < NF_OP_KINDS; ++k) {
      kinds.push_back(k);
      nanos.push_back(0);
      streams.push_back(0);
    }
  } else {
    if (plan->n_nano < 1 || !plan->bounds) {
      err = "plan needs n_nano >= 1 and bounds";
      return NF_E_PLAN;
    }
    g.n_nano = plan->n_nano;
    g.bounds.assign(plan->bounds, plan->bounds + plan->n_nano + 1);
    if (g.bounds.front() != 0 || g.bounds.back() != T) {
      err = fmt("plan bounds must run from 0 to T=%ld", T);
      return NF_E_PLAN;
    }
    for (int32_t j = 0; j < g.n_nano; ++j)
      if (g.bounds[j + 1] <= g.bounds[j]) {
        err = fmt("plan bounds not increasing at nano-batch %ld", j);
        return NF_E_PLAN;
      }
    if (plan->n_streams < 1 || plan->n_streams > 3) {
      err = "plan needs 1..3 streams";
      return NF_E_PLAN;
    }
    g.n_streams = plan->n_streams;
    if (plan->n_ops != NF_OP_KINDS * g.n_nano || !plan->op_kind || !plan->op_nano || !plan->op_stream) {
      err = fmt("plan lists %ld ops, expected %ld", plan->n_ops, NF_OP_KINDS * g.n_nano);
      return NF_E_PLAN;
    }
    std::vector<char> seen(NF_OP_KINDS * g.n_nano, 0);
    for (int32_t i = 0; i < plan->n_ops; ++i) {
      const int32_t k = plan->op_kind[i], j = plan->op_nano[i], s = plan->op_stream[i];
      if (k < 0 || k >= NF_OP_KINDS || j < 0 || j >= g.n_nano || s < 0 || s >= g.n_streams) {
        err = fmt("plan op %ld out of range", i);
        return NF_E_PLAN;
      }
      if (seen[k * g.n_nano + j]++) {
        err = fmt("plan lists op kind %ld of nano-batch %ld twice", k, j);
        return NF_E_PLAN;
      }
      const int32_t lane = plan->op_lane ? plan->op_lane[i] : s;
      if (lane < 0 || lane > 2) {
        err = fmt("plan op %ld: lane out of range 0..2", i);
        return NF_E_PLAN;
      }
      kinds.push_back(k);
      nanos.push_back(j);
      streams.push_back(s);
      lanes.push_back(lane);
    }
  }
  while (g.n_dec < (int32_t)L.req.size() && L.req[g.n_dec].decode) ++g.n_dec;
  // nano-batch of a token row
  auto nano_of = [&](int32_t t) {
    return (int32_t)(std::upper_bound(g.bounds.begin(), g.bounds.end(), t) - g.bounds.begin()) - 1;
  };
  const int32_t n_ops = (int32_t)kinds.size();
  g.ops.resize(n_ops);
  for (int32_t i = 0; i < n_ops; ++i) {
    NanoOp& op = g.ops[i];
    op.kind = kinds[i];
    op.nano = nanos[i];
    op.stream = streams[i];
    const int32_t lo = g.bounds[op.nano], hi = g.bounds[op.nano + 1];
    switch (op.kind) {
      case NF_OP_KQV:
      case NF_OP_O:
      case NF_OP_UGD: op.rows.push_back({lo, hi}); break;
      case NF_OP_DECATTN: {
        // decode requests have one token each and come first: request r = token r
        int32_t r0 = lo, r1 = hi;
        int32_t n_dec = 0;
        while (n_dec < (int32_t)L.req.size() && L.req[n_dec].decode) ++n_dec;
        r0 = std::min(r0, n_dec);
        r1 = std::min(r1, n_dec);
        op.r0 = r0;
        op.r1 = r1;
        if (r1 > r0) op.rows.push_back({r0, r1});
        break;
      }
      case NF_OP_PFATTN: {
        for (int32_t r = 0; r < (int32_t)L.req.size(); ++r) {
          const ReqInfo& ri = L.req[r];
          if (ri.decode) continue;
          if (nano_of(ri.t1 - 1) == op.nano) {
            op.prefill_reqs.push_back(r);
            op.rows.push_back({ri.t0, ri.t1});
          }
        }
        break;
      }
    }
    op.empty = op.rows.empty();
  }
  // dependencies by parent dependency + range intersection
  g.deps.assign(n_ops, {});
  for (int32_t j = 0; j < n_ops; ++j)
    for (int32_t i = 0; i < n_ops; ++i)
      if (i != j && parent_depends(g.ops[i].kind, g.ops[j].kind) && intersects(g.ops[i], g.ops[j]))
        g.deps[j].push_back(i);
  // lane order: an op waits for the lane's previous listed op when that one ran on another
  // stream (on the same stream, stream order already serialises them)
  if (!lanes.empty()) {
    int32_t prev[3] = {-1, -1, -1};
    for (int32_t j = 0; j < n_ops; ++j) {
      const int32_t i = prev[lanes[j]];
      if (i >= 0 && g.ops[i].stream != g.ops[j].stream &&
          std::find(g.deps[j].begin(), g.deps[j].end(), i) == g.deps[j].end())
        g.deps[j].push_back(i);
      prev[lanes[j]] = j;
    }
  }
  // global order: Kahn's algorithm over dependency edges plus per-stream order edges,
  // preferring the plan's listed position
  std::vector<std::vector<int32_t>> succ(n_ops);
  std::vector<int32_t> indeg(n_ops, 0);
  for (int32_t j = 0; j < n_ops; ++j)
    for (int32_t i : g.deps[j]) {
      succ[i].push_back(j);
      indeg[j]++;
    }
  std::vector<int32_t> last(g.n_streams, -1);
  for (int32_t i = 0; i < n_ops; ++i) {
    const int32_t s = g.ops[i].stream;
    if (last[s] >= 0) {
      succ[last[s]].push_back(i);
      indeg[i]++;
    }
    last[s] = i;
  }
  std::vector<char> done(n_ops, 0);
  g.order.clear();
  for (int32_t step = 0; step < n_ops; ++step) {
    int32_t pick = -1;
    for (int32_t i = 0; i < n_ops; ++i)
      if (!done[i] && indeg[i] == 0) {
        pick = i;
        break;
      }
    if (pick < 0) {
      err = "plan order deadlocks: a stream's order contradicts a dependency";
      return NF_E_PLAN;
    }
    done[pick] = 1;
    g.order.push_back(pick);
    for (int32_t j : succ[pick]) indeg[j]--;
  }
  return NF_OK;
}

nf_status build_stack_graph(const PlanGraph& g, int32_t n_layers, bool pipelined, StackGraph& s, std::string& err) {
  s = StackGraph();
  if (n_layers < 1) {
    err = "n_layers must be >= 1";
    return NF_E_ARG;
  }
  const int32_t n = (int32_t)g.ops.size();
  const int32_t N = n_layers * n;
  s.n_layers = n_layers;
  s.n_ops = n;
  s.deps.assign(N, {});
  for (int32_t l = 0; l < n_layers; ++l)
    for (int32_t j = 0; j < n; ++j) {
      auto& d = s.deps[l * n + j];
      for (int32_t i : g.deps[j]) d.push_back(l * n + i);
      if (l > 0 && g.ops[j].kind == NF_OP_KQV)
        for (int32_t i = 0; i < n; ++i)
          if (g.ops[i].kind == NF_OP_UGD && intersects(g.ops[i], g.ops[j])) d.push_back((l - 1) * n + i);
    }
  // listing: layer 0 as listed; every later layer as listed, its KQV ops moved up when
  // pipelined (each right after its last producer in the listing, after any KQV moved
  // there before it)
  s.listing.clear();
  s.listing.reserve(N);
  for (int32_t l = 0; l < n_layers; ++l) {
    for (int32_t j = 0; j < n; ++j)
      if (!(pipelined && l > 0 && g.ops[j].kind == NF_OP_KQV)) s.listing.push_back(l * n + j);
    if (!pipelined || l + 1 >= n_layers) continue;
    // place layer l+1's KQV ops (listed order) inside what is listed so far
    std::vector<int32_t> pos(N, -1);
    for (int32_t k = 0; k < (int32_t)s.listing.size(); ++k) pos[s.listing[k]] = k;
    std::vector<std::pair<int32_t, int32_t>> ins;  // (insert after listing index, op)
    for (int32_t j = 0; j < n; ++j) {
      if (g.ops[j].kind != NF_OP_KQV) continue;
      const int32_t op = (l + 1) * n + j;
      int32_t after = -1;
      for (int32_t d : s.deps[op]) after = std::max(after, pos[d]);
      if (after < 0) after = (int32_t)s.listing.size() - 1;  // no producer: end of layer l
      ins.push_back({after, op});
    }
    std::stable_sort(ins.begin(), ins.end(),
                     [](const std::pair<int32_t, int32_t>& a, const std::pair<int32_t, int32_t>& b) {
                       return a.first < b.first;
                     });
    std::vector<int32_t> merged;
    merged.reserve(s.listing.size() + ins.size());
    size_t q = 0;
    for (size_t k = 0; k < s.listing.size(); ++k) {
      merged.push_back(s.listing[k]);
      while (q < ins.size() && ins[q].first == (int32_t)k) merged.push_back(ins[q++].second);
    }
    s.listing.swap(merged);
  }
  // global order: Kahn's algorithm over dependencies plus per-stream listing order,
  // preferring the earliest listing position
  std::vector<std::vector<int32_t>> succ(N);
  std::vector<int32_t> indeg(N, 0);
  for (int32_t j = 0; j < N; ++j)
    for (int32_t i : s.deps[j]) {
      succ[i].push_back(j);
      indeg[j]++;
    }
  std::vector<int32_t> last(g.n_streams, -1);
  for (int32_t op : s.listing) {
    const int32_t st = g.ops[op % n].stream;
    if (last[st] >= 0) {
      succ[last[st]].push_back(op);
      indeg[op]++;
    }
    last[st] = op;
  }
  std::vector<char> done(N, 0);
  s.order.clear();
  s.order.reserve(N);
  for (int32_t step = 0; step < N; ++step) {
    int32_t pick = -1;
    for (int32_t k = 0; k < N; ++k) {
      const int32_t op = s.listing[k];
      if (!done[op] && indeg[op] == 0) {
        pick = op;
        break;
      }
    }
    if (pick < 0) {
      err = "stack order deadlocks: a stream's order contradicts a dependency";
      return NF_E_PLAN;
    }
    done[pick] = 1;
    s.order.push_back(pick);
    for (int32_t j : succ[pick]) indeg[j]--;
  }
  return NF_OK;
}

nf_status build_kv_moves(const nf_layer_cfg& cfg, const nf_kv_ranges& r, int32_t num_blocks, bool check_alias,
                         std::vector<KvMoveItem>& items, int64_t& n_rows, std::string& err) {
  const int32_t BS = cfg.block_size;
  items.clear();
  n_rows = 0;
  if (r.n_req < 0 || (r.n_req > 0 && (!r.first || !r.n_tokens || !r.block_table || r.max_blocks <= 0))) {
    err = "KV ranges: bad request count or null array";
    return NF_E_ARG;
  }
  std::vector<uint8_t> used;
  if (check_alias) used.assign((size_t)num_blocks * BS, 0);
  for (int32_t q = 0; q < r.n_req; ++q) {
    const int64_t p0 = r.first[q], n = r.n_tokens[q];
    if (p0 < 0 || n < 0) {
      err = fmt("KV range %ld: negative first or length", q);
      return NF_E_ARG;
    }
    if (n == 0) continue;
    if ((p0 + n + BS - 1) / BS > r.max_blocks) {
      err = fmt("KV range %ld needs %ld blocks, table row holds %ld", q, (p0 + n + BS - 1) / BS, r.max_blocks);
      return NF_E_BLOCK_TABLE_SHORT;
    }
    for (int64_t p = p0; p < p0 + n;) {
      const int64_t lb = p / BS;
      const int32_t blk = r.block_table[(size_t)q * r.max_blocks + lb];
      if (blk < 0 || blk >= num_blocks) {
        err = fmt("KV range %ld: block id %ld outside [0, %ld)", q, (int64_t)blk, (int64_t)num_blocks);
        return NF_E_BLOCK_RANGE;
      }
      const int64_t end = std::min(p0 + n, (lb + 1) * BS);
      KvMoveItem it{blk, (int32_t)(p % BS), (int32_t)(end - lb * BS), (int32_t)n_rows};
      if (check_alias)
        for (int32_t o = it.tok0; o < it.tok1; ++o) {
          uint8_t& u = used[(size_t)blk * BS + o];
          if (u) {
            err = fmt("KV range %ld: slot %ld written twice", q, (int64_t)blk * BS + o);
            return NF_E_SLOT_ALIAS;
          }
          u = 1;
        }
      items.push_back(it);
      n_rows += end - p;
      p = end;
    }
  }
  if (n_rows > INT32_MAX) {
    err = "KV ranges: too many tokens";
    return NF_E_ARG;
  }
  return NF_OK;
}

// Chunk size (blocks) for the decode requests [r0, r1): the longest of 128, 64, 32, 16
// blocks that still yields at least kMinUnits (request chunk, KV head) work units, so that
// the waves fill the GPU several times over; long chunks have fewer start-ups and combines
// (70B tensor-parallel share, 1536 requests of 32-256 blocks, one KV head: 128-block chunks
// give 0.825 against 0.830 ms per layer step with 64, and 16-48 are slower still).
static int32_t auto_split(const BatchLayout& L, int32_t r0, int32_t r1, int32_t n_kv) {
  constexpr int64_t kMinUnits = 2048;
  int32_t sp = 128;
  for (; sp > 16; sp /= 2) {
    int64_t units = 0;
    for (int32_t r = r0; r < r1; ++r) units += ((L.req[r].n_keys + 15) / 16 + sp - 1) / sp;
    if (units * n_kv >= kMinUnits) break;
  }
  return sp;
}

// Keys a tile of queries [q0, q1) of a prefill chunk can see: its cached prefix and the
// chunk's queries up to the last one (causal).
static int32_t tile_keys(const PrefillReq& r, int32_t q1) { return r.prefix + q1; }

int prefill_chunk_keys(const std::vector<PrefillReq>& reqs, int n_q, int n_kv) {
  const int G = n_q / n_kv, TQ = prefill_tile_queries(G);
  const int64_t wg_per_item = n_q / prefill_heads_per_wg(G);
  for (int chunk = kPrefillMaxChunkKeys; chunk > 128; chunk /= 2) {
    int64_t items = 0;
    for (const PrefillReq& r : reqs)
      for (int32_t q0 = 0; q0 < r.q_len; q0 += TQ) items += (tile_keys(r, std::min(q0 + TQ, r.q_len)) + chunk - 1) / chunk;
    if (items * wg_per_item >= kPrefillTargetWgs) return chunk;
  }
  return 128;
}

void build_prefill_work(const std::vector<PrefillReq>& reqs, int n_q, int n_kv, int chunk_keys,
                        std::vector<PrefillItem>& items, std::vector<CombineItem>& comb, int32_t& n_parts) {
  const int G = n_q / n_kv, TQ = prefill_tile_queries(G);
  chunk_keys = std::max(32, std::min(chunk_keys, kPrefillMaxChunkKeys)) / 32 * 32;
  const size_t first = items.size();
  for (const PrefillReq& r : reqs)
    for (int32_t q0 = 0; q0 < r.q_len; q0 += TQ) {
      const int32_t q1 = std::min(q0 + TQ, r.q_len);
      const int32_t keys = tile_keys(r, q1);
      // chunks of about equal length in 32-key steps, none empty
      const int32_t steps = (keys + 31) / 32;
      const int32_t per_steps = (steps + (keys + chunk_keys - 1) / chunk_keys - 1) / ((keys + chunk_keys - 1) / chunk_keys);
      const int32_t nch = (steps + per_steps - 1) / per_steps, per = per_steps * 32;
      const int32_t base = nch > 1 ? n_parts : -1;
      for (int32_t c = 0; c < nch; ++c) {
        PrefillItem it{};
        it.req = r.req;
        it.token0 = r.token0;
        it.q_begin = q0;
        it.q_len = r.q_len;
        it.prefix = r.prefix;
        it.key_begin = c * per;
        it.key_end = std::min(keys, (c + 1) * per);
        it.part = nch > 1 ? base + c : -1;
        it.n_chunks = nch;
        items.push_back(it);
      }
      if (nch > 1) {
        for (int32_t i = 0; i < q1 - q0; ++i) comb.push_back(CombineItem{r.token0 + q0 + i, base + i * nch, nch, 0});
        n_parts += (q1 - q0) * nch;
      }
    }
  // longest key ranges first: workgroups start in item order, the shortest last
  std::stable_sort(items.begin() + first, items.end(), [](const PrefillItem& a, const PrefillItem& b) {
    return a.key_end - a.key_begin > b.key_end - b.key_begin;
  });
}

// Work lists of the decode attention and prefill attention nano-ops of each nano-batch.
// split: decode chunk in blocks, 0 = auto_split per nano-op.
void build_work(const BatchLayout& L, const PlanGraph& g, int split, int pf_chunk, int n_q, int n_kv, Meta& M) {
  const int n_nano = g.n_nano;
  M.dec.clear();
  M.comb.clear();
  M.pf.clear();
  M.pcomb.clear();
  M.dec_begin.assign(n_nano + 1, 0);
  M.comb_begin.assign(n_nano + 1, 0);
  M.pf_begin.assign(n_nano + 1, 0);
  M.pcomb_begin.assign(n_nano + 1, 0);
  M.n_parts = 0;
  std::vector<const NanoOp*> dec_op(n_nano, nullptr), pf_op(n_nano, nullptr);
  for (auto& op : g.ops) {
    if (op.kind == NF_OP_DECATTN) dec_op[op.nano] = &op;
    if (op.kind == NF_OP_PFATTN) pf_op[op.nano] = &op;
  }
  for (int j = 0; j < n_nano; ++j) {
    M.dec_begin[j] = (int32_t)M.dec.size();
    M.comb_begin[j] = (int32_t)M.comb.size();
    if (dec_op[j]) {
      const int32_t sp = split > 0 ? split : auto_split(L, dec_op[j]->r0, dec_op[j]->r1, n_kv);
      for (int32_t r = dec_op[j]->r0; r < dec_op[j]->r1; ++r) {
        const ReqInfo& ri = L.req[r];
        const int32_t nblk = (ri.n_keys + 15) / 16;  // KV blocks of 16 tokens
        const int32_t nch = (nblk + sp - 1) / sp;
        const int32_t per = (nblk + nch - 1) / nch;
        for (int32_t c = 0; c < nch; ++c) {
          DecodeItem it;
          it.req = r;
          it.token = ri.t0;
          it.n_keys = ri.n_keys;
          it.blk_begin = c * per;
          it.blk_end = std::min(nblk, (c + 1) * per);
          it.part = nch > 1 ? M.n_parts + c : -1;
          M.dec.push_back(it);
        }
        if (nch > 1) {
          M.comb.push_back(CombineItem{ri.t0, M.n_parts, nch, 0});
          M.n_parts += nch;
        }
      }
      // Longest runs first: workgroups are dispatched in item order as slots free up, so
      // the last ones to start are the shortest and the grid drains evenly (a request of
      // 2048 keys started last would stream alone for a tenth of the kernel). Each item
      // writes its own output row or partial slot, so the order changes no result.
      std::stable_sort(M.dec.begin() + M.dec_begin[j], M.dec.end(), [](const DecodeItem& a, const DecodeItem& b) {
        return a.blk_end - a.blk_begin > b.blk_end - b.blk_begin;
      });
    }
    M.pf_begin[j] = (int32_t)M.pf.size();
    M.pcomb_begin[j] = (int32_t)M.pcomb.size();
    if (pf_op[j]) {
      std::vector<PrefillReq> reqs;
      for (int32_t r : pf_op[j]->prefill_reqs) {
        const ReqInfo& ri = L.req[r];
        reqs.push_back(PrefillReq{r, ri.t0, ri.t1 - ri.t0, ri.cached});
      }
      build_prefill_work(reqs, n_q, n_kv, pf_chunk > 0 ? pf_chunk : prefill_chunk_keys(reqs, n_q, n_kv), M.pf, M.pcomb,
                         M.n_parts);
    }
  }
  M.dec_begin[n_nano] = (int32_t)M.dec.size();
  M.comb_begin[n_nano] = (int32_t)M.comb.size();
  M.pf_begin[n_nano] = (int32_t)M.pf.size();
  M.pcomb_begin[n_nano] = (int32_t)M.pcomb.size();
}


}  // namespace nf

// ---------------------------------------------------------------------------------------
// host-only ABI entry points
// ---------------------------------------------------------------------------------------

static void put_err(char* dst, size_t cap, const std::string& s) {
  if (!dst || cap == 0) return;
  const size_t n = std::min(cap - 1, s.size());
  memcpy(dst, s.data(), n);
  dst[n] = 0;
}

extern "C" nf_status nf_batch_slots(const nf_layer_cfg* cfg, const nf_batch_desc* batch, int32_t num_blocks,
                                    int32_t* pos_out, int32_t* slot_out, char* err_msg, size_t err_cap) {
  std::string err;
  if (!cfg || !batch) {
    put_err(err_msg, err_cap, "null argument");
    return NF_E_ARG;
  }
  nf_status st = nf::check_cfg(*cfg, err);
  nf::BatchLayout L;
  if (st == NF_OK) st = nf::build_layout(*cfg, *batch, num_blocks, L, err);
  if (st != NF_OK) {
    put_err(err_msg, err_cap, err);
    return st;
  }
  if (pos_out) memcpy(pos_out, L.pos.data(), sizeof(int32_t) * L.T);
  if (slot_out) memcpy(slot_out, L.slot.data(), sizeof(int32_t) * L.T);
  put_err(err_msg, err_cap, "");
  return NF_OK;
}

// Token ranges of a batch without a pool (blocks are not needed for the DAG).
static nf_status token_layout(const nf_batch_desc* batch, nf::BatchLayout& L, std::string& err) {
  int64_t t = 0;
  for (int32_t r = 0; r < batch->n_decode + batch->n_prefill; ++r) {
    nf::ReqInfo ri;
    ri.decode = r < batch->n_decode;
    const int32_t q = ri.decode ? 1 : batch->prefill_len[r - batch->n_decode];
    if (q < 1) {
      err = "prefill length < 1";
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
  return NF_OK;
}

static nf_status put_edges(const std::vector<std::vector<int32_t>>& deps, int32_t* edges, int32_t cap,
                           int32_t* n_edges, char* err_msg, size_t err_cap) {
  int32_t n = 0;
  for (int32_t j = 0; j < (int32_t)deps.size(); ++j)
    for (int32_t i : deps[j]) {
      if (n < cap && edges) {
        edges[2 * n] = i;
        edges[2 * n + 1] = j;
      }
      ++n;
    }
  *n_edges = n;
  if (n > cap) {
    put_err(err_msg, err_cap, "edge capacity too small");
    return NF_E_CAPACITY;
  }
  return NF_OK;
}

extern "C" nf_status nf_plan_dependencies(const nf_batch_desc* batch, const nf_plan* plan, int32_t* edges, int32_t cap,
                                          int32_t* n_edges, int32_t* order_out, char* err_msg, size_t err_cap) {
  std::string err;
  if (!batch || !n_edges) {
    put_err(err_msg, err_cap, "null argument");
    return NF_E_ARG;
  }
  nf::BatchLayout L;
  nf_status st = token_layout(batch, L, err);
  if (st == NF_OK) {
    nf::PlanGraph g;
    st = nf::build_plan_graph(L, plan, g, err);
    if (st == NF_OK) {
      if (order_out) memcpy(order_out, g.order.data(), sizeof(int32_t) * g.order.size());
      st = put_edges(g.deps, edges, cap, n_edges, err_msg, err_cap);
      if (st != NF_OK) return st;
    }
  }
  put_err(err_msg, err_cap, err);
  return st;
}

extern "C" nf_status nf_stack_dependencies(const nf_batch_desc* batch, const nf_plan* plan, int32_t n_layers,
                                           int32_t flags, int32_t* edges, int32_t cap, int32_t* n_edges,
                                           int32_t* listing_out, int32_t* order_out, char* err_msg, size_t err_cap) {
  std::string err;
  if (!batch || !n_edges || n_layers < 1 || (flags & ~(NF_STACK_PIPELINE | NF_STACK_GRAPH))) {
    put_err(err_msg, err_cap, "bad argument");
    return NF_E_ARG;
  }
  nf::BatchLayout L;
  nf_status st = token_layout(batch, L, err);
  if (st == NF_OK) {
    nf::PlanGraph g;
    st = nf::build_plan_graph(L, plan, g, err);
    nf::StackGraph sg;
    if (st == NF_OK) st = nf::build_stack_graph(g, n_layers, (flags & NF_STACK_PIPELINE) != 0, sg, err);
    if (st == NF_OK) {
      if (listing_out) memcpy(listing_out, sg.listing.data(), sizeof(int32_t) * sg.listing.size());
      if (order_out) memcpy(order_out, sg.order.data(), sizeof(int32_t) * sg.order.size());
      st = put_edges(sg.deps, edges, cap, n_edges, err_msg, err_cap);
      if (st != NF_OK) return st;
    }
  }
  put_err(err_msg, err_cap, err);
  return st;
}
