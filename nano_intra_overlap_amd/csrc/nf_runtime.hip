// libnanoflow runtime: context, workspaces, batch metadata upload, the nano-operation
// executor and the per-operation entry points.
//
// Executor (NanoFlow OSDI'25 summary page: nano-ops launched as kernels on CUDA streams
// ordered by events; here HIP streams with CU masks): every nano-operation of the plan is
// enqueued on its stream in a global order consistent with each stream's listed order and
// with the range-intersection dependencies; a nano-op waits (hipStreamWaitEvent) on the
// events of the producers it depends on that live on other streams, then records its own
// event. The call forks from the caller's stream through one event and joins back into it.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <map>
#include <memory>
#include <mutex>

#include "nf_batch.h"
#include "nf_internal.h"

using namespace nf;

namespace {

constexpr int kMaxSplit = 4096;    // decode chunk limit (blocks per work item)
constexpr int kDefaultSplit = 0;  // default decode chunk: 0 = chosen per nano-op from its work
constexpr int kMaxStreams = 3;  // + the caller's stream: within the 4 HW queues of a process
// Replay of a captured stack (NF_STACK_GRAPH) is switched off: its first run on the device
// ended in a host segmentation fault inside the capture / instantiate / launch sequence
// below, with no cause found in this library's code. Calls asking for it get
// NF_E_UNSUPPORTED.
constexpr bool kGraphReplayEnabled = false;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct DevBuf {
  void* p = nullptr;
  size_t cap = 0;
};

}  // namespace

// Device scratch of the allocation-free entry point (nf_op_gemm_noalloc): fp32 split-K
// partials live here instead of in a workspace the context allocates. One copy per GPU the
// library runs on, held until the process ends. Host code never uses the symbol itself as
// an address: each device's address is taken once with hipGetSymbolAddress (scratch_setup)
// and kept in g_scratch.
static constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// With `device` current: its address of the scratch array (taken on the first call).
hipError_t scratch_setup(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[device] = p;
  }
  *out = g_scratch[device];
  return hipSuccess;
}
}  // namespace

struct nf_ctx {
  int device = 0;
  std::string err;
  // activation workspace
  DevBuf h, qkv, attn, x1, h2, a;
  // metadata: pinned staging + device copy
  DevBuf meta_dev;
  void* meta_host = nullptr;
  size_t meta_host_cap = 0;
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  // split-KV partials
  DevBuf part_o, part_ml;
  DevBuf gemm_ws;  // split-K fp32 partials, one region per GEMM of a plan
  void* scratch = nullptr;  // this device's address of the static scratch array
  // MoE FFN: per token entry (2 T) the chosen expert, weight, grouped row; per grouped row
  // its token; per nano-batch the expert group table; the grouped expert outputs
  DevBuf moe_idx, moe_out;
  DevBuf kv_stage, kv_items;  // KV offload / reload: token-major staging rows, move items
  void* kv_host = nullptr;     // pinned staging of the move items (their own, so that KV
  size_t kv_host_cap = 0;      // moves on another stream never wait for a layer's upload)
  hipEvent_t kv_upload_done = nullptr;
  bool kv_upload_pending = false;
  size_t moe_rows = 0;  // 2 T the MoE index arrays were laid out for
  uint64_t ws_gen = 0;  // bumped whenever a device buffer is reallocated
  // captured layer stack: its own metadata buffer, the key it was captured for
  hipStream_t cap_stream = nullptr;
  DevBuf graph_meta;
  hipGraph_t graph = nullptr;
  hipGraphExec_t graph_exec = nullptr;
  std::vector<uint64_t> graph_key;
  std::vector<unsigned char> graph_meta_bytes;
  hipEvent_t graph_in = nullptr, graph_out = nullptr;
  int64_t graph_captures = 0, graph_launches = 0;
  // streams keyed by CU mask (all-ones key = unmasked)
  struct StreamEntry {
    std::vector<uint32_t> mask;
    hipStream_t s;
    uint64_t last_use;
  };
  std::vector<StreamEntry> streams;
  uint64_t use_clock = 0;
  std::vector<hipEvent_t> events;
  hipEvent_t fork_ev = nullptr;
  std::vector<hipEvent_t> join_ev;
  int decode_split = kDefaultSplit;
  int prefill_chunk = 0;  // prefill keys per work item (0 = chosen per nano-op)
  int decode_grid = 0;  // max workgroups of the decode attention kernel (0 = one wave per work unit)
  int decode_nbuf = 0;  // KV blocks per online-softmax step (0: chosen per launch from its work)
  int decode_ring = 0;  // register buffers of decode_nbuf blocks; decode_ring - 1 groups in flight
  int gemm_variant[NF_OP_KINDS][2];  // per dense op kind: [0] first GEMM, [1] second (UGD down); -1 = default
  // kernel timing: events recorded around instrumented kernel classes on their own stream
  uint32_t timing_mask = 0;
  struct TimedLaunch {
    int32_t cls;
    hipEvent_t start, stop;
  };
  std::vector<TimedLaunch> timed;
  std::vector<hipEvent_t> timing_pool;  // timing-enabled events, reused
  size_t timing_pool_used = 0;
};

namespace {

nf_status hip_fail(nf_ctx* ctx, hipError_t e, const char* what) {
  ctx->err = std::string(what) + ": " + hipGetErrorString(e);
  return NF_E_HIP;
}

#define NF_HIP(ctx, expr)                                   \
  do {                                                      \
    hipError_t e_ = (expr);                                 \
    if (e_ != hipSuccess) return hip_fail((ctx), e_, #expr); \
  } while (0)

nf_status ensure(nf_ctx* ctx, DevBuf& b, size_t bytes) {
  if (b.cap >= bytes) return NF_OK;
  if (b.p) {
    NF_HIP(ctx, hipDeviceSynchronize());
    NF_HIP(ctx, hipFree(b.p));
    b.p = nullptr;
    b.cap = 0;
  }
  const size_t cap = align_up(std::max<size_t>(bytes, 256), 1 << 20);
  NF_HIP(ctx, hipMalloc(&b.p, cap));
  b.cap = cap;
  ++ctx->ws_gen;
  return NF_OK;
}

nf_status ensure_host(nf_ctx* ctx, size_t bytes) {
  if (ctx->meta_host_cap >= bytes) return NF_OK;
  if (ctx->upload_pending) {
    NF_HIP(ctx, hipEventSynchronize(ctx->upload_done));
    ctx->upload_pending = false;
  }
  if (ctx->meta_host) NF_HIP(ctx, hipHostFree(ctx->meta_host));
  ctx->meta_host = nullptr;
  const size_t cap = align_up(bytes, 1 << 20);
  NF_HIP(ctx, hipHostMalloc(&ctx->meta_host, cap, hipHostMallocDefault));
  ctx->meta_host_cap = cap;
  return NF_OK;
}

// Stream for a CU mask (nullptr mask = whole GPU). Masks must give each XCD the same
// non-zero number of CUs.
nf_status mask_ok(nf_ctx* ctx, const uint32_t* m) {
  int per[kNumXcd] = {0};
  for (int i = 0; i < NF_CU_MASK_WORDS * 32; ++i)
    if (m[i / 32] >> (i % 32) & 1u) per[i % kNumXcd]++;
  for (int x = 0; x < kNumXcd; ++x)
    if (per[x] == 0 || per[x] != per[0]) {
      char buf[160];
      snprintf(buf, sizeof buf, "CU mask gives XCD %d %d CUs and XCD 0 %d; every XCD needs the same non-zero count",
               x, per[x], per[0]);
      ctx->err = buf;
      return NF_E_CU_MASK;
    }
  return NF_OK;
}

// Streams are cached per (mask, plan stream index): plan streams are always distinct
// streams, masked or not.
nf_status get_stream(nf_ctx* ctx, const uint32_t* mask, int idx, hipStream_t* out) {
  std::vector<uint32_t> key(NF_CU_MASK_WORDS, 0xFFFFFFFFu);
  if (mask) key.assign(mask, mask + NF_CU_MASK_WORDS);
  key.push_back((uint32_t)idx);
  for (auto& e : ctx->streams)
    if (e.mask == key) {
      e.last_use = ++ctx->use_clock;
      *out = e.s;
      return NF_OK;
    }
  if (mask) {
    nf_status st = mask_ok(ctx, mask);
    if (st != NF_OK) return st;
  }
  if ((int)ctx->streams.size() >= kMaxStreams) {
    // evict the least recently used stream (its work completes before destruction)
    auto it = std::min_element(ctx->streams.begin(), ctx->streams.end(),
                               [](const nf_ctx::StreamEntry& a, const nf_ctx::StreamEntry& b) {
                                 return a.last_use < b.last_use;
                               });
    NF_HIP(ctx, hipStreamSynchronize(it->s));
    NF_HIP(ctx, hipStreamDestroy(it->s));
    ctx->streams.erase(it);
  }
  hipStream_t s;
  if (mask) {
    NF_HIP(ctx, hipExtStreamCreateWithCUMask(&s, NF_CU_MASK_WORDS, mask));
  } else {
    NF_HIP(ctx, hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  }
  ctx->streams.push_back({key, s, ++ctx->use_clock});
  *out = s;
  return NF_OK;
}

// Events that order work between streams of this one device: agent-scope fences suffice
// (every stream's kernels run on this device), so the system-scope fence that would make
// memory visible to the host at each record is left out.
constexpr unsigned kDeviceEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

nf_status ensure_events(nf_ctx* ctx, size_t n) {
  while (ctx->events.size() < n) {
    hipEvent_t e;
    NF_HIP(ctx, hipEventCreateWithFlags(&e, kDeviceEventFlags));
    ctx->events.push_back(e);
  }
  while (ctx->join_ev.size() < (size_t)kMaxStreams) {
    hipEvent_t e;
    NF_HIP(ctx, hipEventCreateWithFlags(&e, kDeviceEventFlags));
    ctx->join_ev.push_back(e);
  }
  return NF_OK;
}

// ---------------------------------------------------------------------------------------
// metadata
// ---------------------------------------------------------------------------------------

// Byte offsets of the packed metadata (one upload per call).
struct MetaPack {
  size_t o_pos = 0, o_slot = 0, o_inv = 0, o_dec = 0, o_comb = 0, o_pcomb = 0, o_pf = 0, o_bt = 0, total = 0;
  bool bt_up = false;
};

// Pack the metadata into the pinned staging buffer (after the previous upload from it).
nf_status pack_meta(nf_ctx* ctx, const nf_layer_cfg& cfg, const nf_batch_desc& b, const BatchLayout& L, const Meta& M,
                    MetaPack& P) {
  const int T = L.T;
  const int half = cfg.head_dim / 2;
  const size_t n_req = L.req.size();
  P = MetaPack();
  P.bt_up = b.block_table_dev == nullptr;
  size_t off = 0;
  auto slot = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  P.o_pos = slot(sizeof(int32_t) * T);
  P.o_slot = slot(sizeof(int32_t) * T);
  P.o_inv = slot(sizeof(float) * half);
  P.o_dec = slot(sizeof(DecodeItem) * M.dec.size());
  P.o_comb = slot(sizeof(CombineItem) * M.comb.size());
  P.o_pcomb = slot(sizeof(CombineItem) * M.pcomb.size());
  P.o_pf = slot(sizeof(PrefillItem) * M.pf.size());
  P.o_bt = slot(P.bt_up ? sizeof(int32_t) * n_req * b.max_blocks : 0);
  P.total = off;
  nf_status st = ensure_host(ctx, P.total);
  if (st != NF_OK) return st;
  if (ctx->upload_pending) {
    NF_HIP(ctx, hipEventSynchronize(ctx->upload_done));  // staging buffer free again
    ctx->upload_pending = false;
  }
  unsigned char* h = static_cast<unsigned char*>(ctx->meta_host);
  memset(h, 0, P.total);  // padding too: the bytes are compared when a graph is reused
  memcpy(h + P.o_pos, L.pos.data(), sizeof(int32_t) * T);
  memcpy(h + P.o_slot, L.slot.data(), sizeof(int32_t) * T);
  float* inv = reinterpret_cast<float*>(h + P.o_inv);
  for (int i = 0; i < half; ++i) inv[i] = (float)std::pow((double)cfg.rope_base, -2.0 * i / cfg.head_dim);
  if (!M.dec.empty()) memcpy(h + P.o_dec, M.dec.data(), sizeof(DecodeItem) * M.dec.size());
  if (!M.comb.empty()) memcpy(h + P.o_comb, M.comb.data(), sizeof(CombineItem) * M.comb.size());
  if (!M.pcomb.empty()) memcpy(h + P.o_pcomb, M.pcomb.data(), sizeof(CombineItem) * M.pcomb.size());
  if (!M.pf.empty()) memcpy(h + P.o_pf, M.pf.data(), sizeof(PrefillItem) * M.pf.size());
  if (P.bt_up && n_req) memcpy(h + P.o_bt, b.block_table, sizeof(int32_t) * n_req * b.max_blocks);
  return NF_OK;
}

// Copy the staged metadata to `dst` on `stream` (ordered before the work that reads it).
nf_status copy_meta(nf_ctx* ctx, const MetaPack& P, DevBuf& dst, hipStream_t stream) {
  if (dst.cap < P.total) {
    nf_status st = ensure(ctx, dst, P.total);
    if (st != NF_OK) return st;
  }
  NF_HIP(ctx, hipMemcpyAsync(dst.p, ctx->meta_host, P.total, hipMemcpyHostToDevice, stream));
  NF_HIP(ctx, hipEventRecord(ctx->upload_done, stream));
  ctx->upload_pending = true;
  return NF_OK;
}

// Device pointers of the metadata held at `base`.
void point_meta(const MetaPack& P, const void* base, const nf_batch_desc& b, Meta& M) {
  const unsigned char* d = static_cast<const unsigned char*>(base);
  M.d_pos = reinterpret_cast<const int32_t*>(d + P.o_pos);
  M.d_slot = reinterpret_cast<const int32_t*>(d + P.o_slot);
  M.d_inv_freq = reinterpret_cast<const float*>(d + P.o_inv);
  M.d_dec = reinterpret_cast<const DecodeItem*>(d + P.o_dec);
  M.d_comb = reinterpret_cast<const CombineItem*>(d + P.o_comb);
  M.d_pcomb = reinterpret_cast<const CombineItem*>(d + P.o_pcomb);
  M.d_pf = reinterpret_cast<const PrefillItem*>(d + P.o_pf);
  M.d_bt = P.bt_up ? reinterpret_cast<const int32_t*>(d + P.o_bt) : b.block_table_dev;
}

// Pack and upload the metadata to the context's metadata buffer on `stream`.
nf_status upload_meta(nf_ctx* ctx, const nf_layer_cfg& cfg, const nf_batch_desc& b, const BatchLayout& L, Meta& M,
                      hipStream_t stream) {
  MetaPack P;
  nf_status st = pack_meta(ctx, cfg, b, L, M, P);
  if (st != NF_OK) return st;
  if ((st = copy_meta(ctx, P, ctx->meta_dev, stream)) != NF_OK) return st;
  point_meta(P, ctx->meta_dev.p, b, M);
  return NF_OK;
}

nf_status ensure_parts(nf_ctx* ctx, const nf_layer_cfg& cfg, int32_t n_parts) {
  const int G = cfg.n_q_heads / cfg.n_kv_heads;
  const size_t n = (size_t)std::max(n_parts, 1) * cfg.n_kv_heads * G;
  nf_status st = ensure(ctx, ctx->part_o, n * cfg.head_dim * sizeof(float));
  if (st != NF_OK) return st;
  return ensure(ctx, ctx->part_ml, n * 2 * sizeof(float));
}

// MoE index arrays in ctx->moe_idx for 2T token entries: sel | wts | pos | src | group
// tables (2 n_experts per nano-batch, room for T nano-batches).
struct MoeIdx {
  int32_t* sel;
  float* wts;
  int32_t* pos;
  int32_t* src;
  int32_t* grp;
};
MoeIdx moe_idx(nf_ctx* ctx) {
  const size_t n = ctx->moe_rows;
  char* b = static_cast<char*>(ctx->moe_idx.p);
  return MoeIdx{reinterpret_cast<int32_t*>(b), reinterpret_cast<float*>(b + 4 * n),
                reinterpret_cast<int32_t*>(b + 8 * n), reinterpret_cast<int32_t*>(b + 12 * n),
                reinterpret_cast<int32_t*>(b + 16 * n)};
}

nf_status ensure_workspace(nf_ctx* ctx, const nf_layer_cfg& c, int T) {
  const size_t t = std::max(T, 1);
  const size_t qkvw = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t fan = c.n_experts > 0 ? (size_t)c.top_k : 1;  // rows of a per token
  nf_status st;
  if ((st = ensure(ctx, ctx->h, t * c.hidden * 2)) != NF_OK) return st;
  if ((st = ensure(ctx, ctx->qkv, t * qkvw * 2)) != NF_OK) return st;
  if ((st = ensure(ctx, ctx->attn, t * c.n_q_heads * c.head_dim * 2)) != NF_OK) return st;
  if ((st = ensure(ctx, ctx->x1, t * c.hidden * 2)) != NF_OK) return st;
  if ((st = ensure(ctx, ctx->h2, t * c.hidden * 2)) != NF_OK) return st;
  if ((st = ensure(ctx, ctx->a, fan * t * c.ffn * 2)) != NF_OK) return st;
  if (c.n_experts > 0) {
    const size_t rows = 2 * t;
    if ((st = ensure(ctx, ctx->moe_out, rows * c.hidden * 2)) != NF_OK) return st;
    // laid out for the most rows seen so far; group tables for up to rows / 2 nano-batches
    const size_t r = std::max(rows, ctx->moe_rows);
    const size_t need = 16 * r + 4 * (size_t)(2 * c.n_experts) * (r / 2);
    if (ctx->moe_rows < r || ctx->moe_idx.cap < need) {
      if ((st = ensure(ctx, ctx->moe_idx, need)) != NF_OK) return st;
      ctx->moe_rows = r;
    }
  }
  return NF_OK;
}

// ---------------------------------------------------------------------------------------
// nano-operation launch
// ---------------------------------------------------------------------------------------

struct LayerArgs {
  const nf_layer_cfg* cfg;
  const nf_layer_weights* w;
  const bf16* x;
  bf16* y;
  nf_kv_pool* pool;
  int max_blocks;
  int decode_grid;
};

int pick_variant(nf_ctx* ctx, int kind, int which, int m, int n, int k, int epi) {
  const int v = ctx->gemm_variant[kind][which];
  if (gemm_variant_supported(v, m, n, k, epi)) return v;
  return gemm_default_variant(m, n, k, epi);
}

// Split-K workspace of every GEMM of the plan, each in a region of its own (GEMMs of one
// plan may run concurrently on different streams).
nf_status plan_gemm_ws(nf_ctx* ctx, const nf_layer_cfg& c, const PlanGraph& g, Meta& M) {
  const int H = c.hidden, F = c.ffn, Q = c.n_q_heads * c.head_dim;
  const int W = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  M.gemm_ws_off.assign(2 * g.ops.size(), 0);
  size_t total = 0;
  auto take = [&](size_t i, size_t bytes) {
    if (!bytes) return;
    M.gemm_ws_off[i] = total;
    total += (bytes + 255) / 256 * 256;
  };
  for (size_t i = 0; i < g.ops.size(); ++i) {
    const NanoOp& op = g.ops[i];
    const int m = g.bounds[op.nano + 1] - g.bounds[op.nano];
    if (m <= 0) continue;
    if (op.kind == NF_OP_KQV) take(2 * i, gemm_workspace_bytes(pick_variant(ctx, NF_OP_KQV, 0, m, W, H, 0), m, W));
    if (op.kind == NF_OP_O) take(2 * i, gemm_workspace_bytes(pick_variant(ctx, NF_OP_O, 0, m, H, Q, 1), m, H));
    if (op.kind == NF_OP_UGD && c.n_experts == 0) {
      take(2 * i, gemm_workspace_bytes(pick_variant(ctx, NF_OP_UGD, 0, m, F, H, 2), m, F));
      take(2 * i + 1, gemm_workspace_bytes(pick_variant(ctx, NF_OP_UGD, 1, m, H, F, 1), m, H));
    }
  }
  return total ? ensure(ctx, ctx->gemm_ws, total) : NF_OK;
}

nf_status timing_event(nf_ctx* ctx, hipEvent_t* e) {
  if (ctx->timing_pool_used == ctx->timing_pool.size()) {
    hipEvent_t ev;  // timing only: no memory is handed to the host through it
    NF_HIP(ctx, hipEventCreateWithFlags(&ev, hipEventDisableSystemFence));
    ctx->timing_pool.push_back(ev);
  }
  *e = ctx->timing_pool[ctx->timing_pool_used++];
  return NF_OK;
}

// Launch `fn` on stream s, bracketed by timing events when its class is instrumented.
template <class F>
nf_status timed(nf_ctx* ctx, int cls, hipStream_t s, F fn) {
  const bool on = (ctx->timing_mask >> cls) & 1u;
  hipEvent_t a = nullptr, b = nullptr;
  if (on) {
    nf_status st = timing_event(ctx, &a);
    if (st == NF_OK) st = timing_event(ctx, &b);
    if (st != NF_OK) return st;
    NF_HIP(ctx, hipEventRecord(a, s));
  }
  NF_HIP(ctx, fn());
  if (on) {
    NF_HIP(ctx, hipEventRecord(b, s));
    ctx->timed.push_back({cls, a, b});
  }
  return NF_OK;
}

// As timed, for a launcher that records the events in its kernel's dispatch (fn(start,
// stop), both null when the class is not timed): no marker packets on the stream, so timing
// does not delay the kernels around it.
template <class F>
nf_status timed_dispatch(nf_ctx* ctx, int cls, F fn) {
  const bool on = (ctx->timing_mask >> cls) & 1u;
  hipEvent_t a = nullptr, b = nullptr;
  if (on) {
    nf_status st = timing_event(ctx, &a);
    if (st == NF_OK) st = timing_event(ctx, &b);
    if (st != NF_OK) return st;
  }
  NF_HIP(ctx, fn(a, b));
  if (on) ctx->timed.push_back({cls, a, b});
  return NF_OK;
}

int pick_grouped(nf_ctx* ctx, int which, int rows, int n_experts, int n, int k, int epi) {
  const int v = ctx->gemm_variant[NF_OP_UGD][which];
  if (gemm_grouped_variant_ok(v, n, k, epi)) return v;
  return gemm_grouped_default_variant(rows, n_experts, k, epi);
}

// MoE FFN over token rows [lo, hi): y = x1 + sum_k w_k expert_k(h2); grp is this
// nano-batch's group table. The token entries of [lo, hi) own grouped rows [2 lo, 2 hi).
nf_status moe_ffn_rows(nf_ctx* ctx, const nf_layer_cfg& c, const nf_layer_weights& w, const bf16* h2, const bf16* x1,
                       bf16* y, int lo, int hi, int32_t* grp, hipStream_t s) {
  const int H = c.hidden, F = c.ffn, E = c.n_experts, rows = 2 * (hi - lo);
  const MoeIdx ix = moe_idx(ctx);
  bf16* a = static_cast<bf16*>(ctx->a.p) + (size_t)2 * lo * F;
  bf16* out = static_cast<bf16*>(ctx->moe_out.p) + (size_t)2 * lo * H;
  nf_status st;
  if ((st = timed(ctx, NF_K_MOE_ROUTE, s, [&] {
         return launch_moe_route(h2, static_cast<const bf16*>(w.w_router), lo, hi, H, E, ix.sel, ix.wts, ix.pos,
                                 ix.src, grp, s);
       })) != NF_OK)
    return st;
  if ((st = timed(ctx, NF_K_GEMM_UG, s, [&] {
         return launch_gemm_grouped(h2, ix.src + 2 * lo, static_cast<const bf16*>(w.w_gate_up), (long long)2 * F * H, a,
                                    grp, E, rows, F, H, 2, pick_grouped(ctx, 0, rows, E, F, H, 2), s);
       })) != NF_OK)
    return st;
  if ((st = timed(ctx, NF_K_GEMM_DOWN, s, [&] {
         return launch_gemm_grouped(a, nullptr, static_cast<const bf16*>(w.w_down), (long long)H * F, out, grp, E, rows,
                                    H, F, 0, pick_grouped(ctx, 1, rows, E, H, F, 0), s);
       })) != NF_OK)
    return st;
  return timed(ctx, NF_K_MOE_COMBINE, s,
               [&] { return launch_moe_combine(x1, out - (size_t)2 * lo * H, ix.pos, ix.wts, y, lo, hi, H, s); });
}

nf_status launch_op(nf_ctx* ctx, const LayerArgs& A, const PlanGraph& g, const NanoOp& op, const Meta& M,
                    hipStream_t s) {
  const nf_layer_cfg& c = *A.cfg;
  const int H = c.hidden, F = c.ffn, d = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int W = (nq + 2 * nkv) * d;
  const int lo = g.bounds[op.nano], hi = g.bounds[op.nano + 1], m = hi - lo;
  const size_t op_i = &op - g.ops.data();
  auto ws = [&](int which) {
    return reinterpret_cast<float*>(static_cast<char*>(ctx->gemm_ws.p) + M.gemm_ws_off[2 * op_i + which]);
  };
  const size_t ws_cap = ctx->gemm_ws.cap;
  bf16* h = static_cast<bf16*>(ctx->h.p);
  bf16* qkv = static_cast<bf16*>(ctx->qkv.p);
  bf16* attn = static_cast<bf16*>(ctx->attn.p);
  bf16* x1 = static_cast<bf16*>(ctx->x1.p);
  bf16* h2 = static_cast<bf16*>(ctx->h2.p);
  bf16* a = static_cast<bf16*>(ctx->a.p);
  const bf16* const* wp = nullptr;
  (void)wp;
  nf_status st = NF_OK;
#define NF_TRY(expr)              \
  do {                            \
    if ((st = (expr)) != NF_OK) return st; \
  } while (0)
  switch (op.kind) {
    case NF_OP_KQV: {
      NF_TRY(timed(ctx, NF_K_RMSNORM, s, [&] {
        return launch_rmsnorm(A.x + (size_t)lo * H, static_cast<const bf16*>(A.w->g_attn), h + (size_t)lo * H, m, H,
                              c.rms_eps, s);
      }));
      NF_TRY(timed(ctx, NF_K_GEMM_KQV, s, [&] {
        return launch_gemm(h + (size_t)lo * H, static_cast<const bf16*>(A.w->w_qkv), qkv + (size_t)lo * W, nullptr, m,
                           W, H, 0, pick_variant(ctx, NF_OP_KQV, 0, m, W, H, 0), s, ws(0), ws_cap - M.gemm_ws_off[2 * op_i]);
      }));
      // decode tokens' K/V go to the pool after their attention (DECATTN below): an attention
      // launch right after the partial-line stores of their append ran 3-6% slower
      NF_TRY(timed(ctx, NF_K_ROPE_KV, s, [&] {
        return launch_rope_kv(qkv, M.d_pos, M.d_slot, M.d_inv_freq, static_cast<bf16*>(A.pool->k),
                              static_cast<bf16*>(A.pool->v), lo, hi, nq, nkv, d, s, g.n_dec);
      }));
      break;
    }
    case NF_OP_DECATTN: {
      const int i0 = M.dec_begin[op.nano], i1 = M.dec_begin[op.nano + 1];
      const int c0 = M.comb_begin[op.nano], c1 = M.comb_begin[op.nano + 1];
      NF_TRY(timed_dispatch(ctx, NF_K_DECODE_ATTN, [&](hipEvent_t e0, hipEvent_t e1) {
        return launch_decode_attn(qkv, static_cast<const bf16*>(A.pool->k), static_cast<const bf16*>(A.pool->v),
                                  M.d_bt, A.max_blocks, M.d_dec + i0, i1 - i0, static_cast<float*>(ctx->part_o.p),
                                  static_cast<float*>(ctx->part_ml.p), attn, nq, nkv, d, A.decode_grid,
                                  ctx->decode_nbuf, ctx->decode_ring, s, e0, e1, /*new_from_qkv=*/1);
      }));
      if (c1 > c0)
        NF_TRY(timed(ctx, NF_K_DECODE_COMBINE, s, [&] {
          return launch_decode_combine(M.d_comb + c0, c1 - c0, static_cast<const float*>(ctx->part_o.p),
                                       static_cast<const float*>(ctx->part_ml.p), attn, nq, nkv, d, s);
        }));
      // the decode tokens' K/V (rotated k and v in qkv) into their pool slots
      NF_TRY(timed(ctx, NF_K_ROPE_KV, s, [&] {
        return launch_kv_append(qkv, M.d_slot, static_cast<bf16*>(A.pool->k), static_cast<bf16*>(A.pool->v), op.r0,
                                op.r1, nq, nkv, d, s);
      }));
      break;
    }
    case NF_OP_PFATTN: {
      const int i0 = M.pf_begin[op.nano], i1 = M.pf_begin[op.nano + 1];
      const int c0 = M.pcomb_begin[op.nano], c1 = M.pcomb_begin[op.nano + 1];
      NF_TRY(timed(ctx, NF_K_PREFILL_ATTN, s, [&] {
        return launch_prefill_attn(qkv, static_cast<const bf16*>(A.pool->k), static_cast<const bf16*>(A.pool->v),
                                   M.d_bt, A.max_blocks, M.d_pf + i0, i1 - i0, M.d_pcomb + c0, c1 - c0,
                                   static_cast<float*>(ctx->part_o.p), static_cast<float*>(ctx->part_ml.p), attn, nq,
                                   nkv, d, s);
      }));
      break;
    }
    case NF_OP_O: {
      NF_TRY(timed(ctx, NF_K_GEMM_O, s, [&] {
        return launch_gemm(attn + (size_t)lo * nq * d, static_cast<const bf16*>(A.w->w_o), x1 + (size_t)lo * H,
                           A.x + (size_t)lo * H, m, H, nq * d, 1, pick_variant(ctx, NF_OP_O, 0, m, H, nq * d, 1), s,
                           ws(0), ws_cap - M.gemm_ws_off[2 * op_i]);
      }));
      break;
    }
    case NF_OP_UGD: {
      NF_TRY(timed(ctx, NF_K_RMSNORM, s, [&] {
        return launch_rmsnorm(x1 + (size_t)lo * H, static_cast<const bf16*>(A.w->g_ffn), h2 + (size_t)lo * H, m, H,
                              c.rms_eps, s);
      }));
      if (c.n_experts > 0) {
        NF_TRY(moe_ffn_rows(ctx, c, *A.w, h2, x1, A.y, lo, hi, moe_idx(ctx).grp + (size_t)op.nano * 2 * c.n_experts,
                            s));
        break;
      }
      NF_TRY(timed(ctx, NF_K_GEMM_UG, s, [&] {
        return launch_gemm(h2 + (size_t)lo * H, static_cast<const bf16*>(A.w->w_gate_up), a + (size_t)lo * F, nullptr,
                           m, F, H, 2, pick_variant(ctx, NF_OP_UGD, 0, m, F, H, 2), s, ws(0),
                           ws_cap - M.gemm_ws_off[2 * op_i]);
      }));
      NF_TRY(timed(ctx, NF_K_GEMM_DOWN, s, [&] {
        return launch_gemm(a + (size_t)lo * F, static_cast<const bf16*>(A.w->w_down), A.y + (size_t)lo * H,
                           x1 + (size_t)lo * H, m, H, F, 1, pick_variant(ctx, NF_OP_UGD, 1, m, H, F, 1), s, ws(1),
                           ws_cap - M.gemm_ws_off[2 * op_i + 1]);
      }));
      break;
    }
  }
#undef NF_TRY
  return NF_OK;
}

// Everything of a call before the metadata upload: validation, layout, DAG, work lists and
// workspace sizes (may reallocate context buffers; enqueues nothing).
nf_status prepare_host(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_batch_desc* batch, int32_t num_blocks,
                       const nf_plan* plan, BatchLayout& L, PlanGraph& g, Meta& M) {
  nf_status st = check_cfg(*cfg, ctx->err);
  if (st != NF_OK) return st;
  st = build_layout(*cfg, *batch, num_blocks, L, ctx->err);
  if (st != NF_OK) return st;
  st = build_plan_graph(L, plan, g, ctx->err);
  if (st != NF_OK) return st;
  if (plan && plan->cu_masks)
    for (int s = 0; s < plan->n_streams; ++s) {
      st = mask_ok(ctx, plan->cu_masks + s * NF_CU_MASK_WORDS);
      if (st != NF_OK) return st;
    }
  build_work(L, g, ctx->decode_split, ctx->prefill_chunk, cfg->n_q_heads, cfg->n_kv_heads, M);
  if ((st = ensure_workspace(ctx, *cfg, L.T)) != NF_OK) return st;
  if ((st = ensure_parts(ctx, *cfg, M.n_parts)) != NF_OK) return st;
  return plan_gemm_ws(ctx, *cfg, g, M);
}

nf_status prepare_batch(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_batch_desc* batch, int32_t num_blocks,
                        const nf_plan* plan, BatchLayout& L, PlanGraph& g, Meta& M, hipStream_t stream) {
  nf_status st = prepare_host(ctx, cfg, batch, num_blocks, plan, L, g, M);
  if (st != NF_OK) return st;
  return upload_meta(ctx, *cfg, *batch, L, M, stream);
}

// The layers of one call: layer l reads x (layer 0: x_in, later layers: y in place).
struct StackArgs {
  const nf_layer_cfg* cfg;
  int32_t n_layers;
  const nf_layer_weights* w;  // [n_layers]
  const bf16* x_in;
  bf16* y;
  nf_kv_pool* pools;  // [n_layers]
  int max_blocks;
  int decode_grid;
  LayerArgs layer(int l) const {
    return LayerArgs{cfg, &w[l], l == 0 ? x_in : y, y, &pools[l], max_blocks, decode_grid};
  }
};

// One nano-batch on one unmasked stream: nothing to order across streams, so the caller's
// stream runs it directly (no fork/join).
bool runs_direct(const nf_plan* plan, const PlanGraph& g) {
  return !plan || (g.n_streams == 1 && !plan->cu_masks);
}

// The plan's streams and enough events, created before anything is enqueued (a capture
// then sees no creation calls).
nf_status plan_resources(nf_ctx* ctx, const nf_plan* plan, const PlanGraph& g, size_t n_stack_ops,
                         std::vector<hipStream_t>& ss) {
  ss.clear();
  if (runs_direct(plan, g)) return NF_OK;
  ss.resize(g.n_streams);
  for (int s = 0; s < g.n_streams; ++s) {
    nf_status st = get_stream(ctx, plan->cu_masks ? plan->cu_masks + s * NF_CU_MASK_WORDS : nullptr, s, &ss[s]);
    if (st != NF_OK) return st;
  }
  return ensure_events(ctx, n_stack_ops);
}

// Enqueue every nano-op of the stack in the graph's global order: directly on `caller`
// when `ss` is empty, else on the plan's streams, forked from and joined back into `caller`.
nf_status enqueue_stack(nf_ctx* ctx, const StackArgs& S, const PlanGraph& g, const StackGraph& sg, const Meta& M,
                        const std::vector<hipStream_t>& ss, hipStream_t caller) {
  const int32_t n = sg.n_ops;
  nf_status st;
  if (ss.empty()) {
    for (int32_t op : sg.order) {
      const NanoOp& o = g.ops[op % n];
      if (o.empty && o.kind != NF_OP_KQV) continue;
      if ((st = launch_op(ctx, S.layer(op / n), g, o, M, caller)) != NF_OK) return st;
    }
    return NF_OK;
  }
  // an op's completion event is recorded only when an op on another stream waits for it
  const size_t N = sg.order.size();
  std::vector<char> waited(N, 0);
  for (size_t j = 0; j < N; ++j)
    for (int32_t dep : sg.deps[j])
      if (g.ops[dep % n].stream != g.ops[j % n].stream) waited[dep] = 1;
  NF_HIP(ctx, hipEventRecord(ctx->fork_ev, caller));
  std::vector<char> used(g.n_streams, 0);
  for (auto& op : g.ops) used[op.stream] = 1;
  for (int s = 0; s < g.n_streams; ++s)
    if (used[s]) NF_HIP(ctx, hipStreamWaitEvent(ss[s], ctx->fork_ev, 0));
  for (int32_t i : sg.order) {
    const NanoOp& op = g.ops[i % n];
    hipStream_t s = ss[op.stream];
    for (int32_t dep : sg.deps[i])
      if (g.ops[dep % n].stream != op.stream) NF_HIP(ctx, hipStreamWaitEvent(s, ctx->events[dep], 0));
    if (!op.empty || op.kind == NF_OP_KQV)
      if ((st = launch_op(ctx, S.layer(i / n), g, op, M, s)) != NF_OK) return st;
    if (waited[i]) NF_HIP(ctx, hipEventRecord(ctx->events[i], s));
  }
  for (int s = 0; s < g.n_streams; ++s)
    if (used[s]) {
      NF_HIP(ctx, hipEventRecord(ctx->join_ev[s], ss[s]));
      NF_HIP(ctx, hipStreamWaitEvent(caller, ctx->join_ev[s], 0));
    }
  return NF_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// ABI
// ---------------------------------------------------------------------------------------

extern "C" const char* nf_version(void) { return "nanoflow-mi355x 0.1"; }

extern "C" nf_status nf_ctx_create(int device, nf_ctx** out) {
  if (!out) return NF_E_ARG;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return NF_E_ARG;
  if (hipSetDevice(device) != hipSuccess) return NF_E_HIP;
  std::unique_ptr<nf_ctx> ctx(new nf_ctx());
  ctx->device = device;
  for (auto& row : ctx->gemm_variant) row[0] = row[1] = -1;
  if (hipEventCreateWithFlags(&ctx->upload_done, hipEventDisableTiming) != hipSuccess) return NF_E_HIP;
  if (hipEventCreateWithFlags(&ctx->fork_ev, kDeviceEventFlags) != hipSuccess) return NF_E_HIP;
  if (device >= kMaxDevices || scratch_setup(device, &ctx->scratch) != hipSuccess) return NF_E_HIP;
  if (gemm_prepare_kernels() != hipSuccess) return NF_E_HIP;
  *out = ctx.release();
  return NF_OK;
}

extern "C" void nf_ctx_destroy(nf_ctx* ctx) {
  if (!ctx) return;
  (void)hipSetDevice(ctx->device);
  (void)hipDeviceSynchronize();
  for (auto& e : ctx->streams) (void)hipStreamDestroy(e.s);
  for (auto e : ctx->events) (void)hipEventDestroy(e);
  for (auto e : ctx->timing_pool) (void)hipEventDestroy(e);
  for (auto e : ctx->join_ev) (void)hipEventDestroy(e);
  if (ctx->fork_ev) (void)hipEventDestroy(ctx->fork_ev);
  if (ctx->graph_exec) (void)hipGraphExecDestroy(ctx->graph_exec);
  if (ctx->graph) (void)hipGraphDestroy(ctx->graph);
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  if (ctx->graph_in) (void)hipEventDestroy(ctx->graph_in);
  if (ctx->graph_out) (void)hipEventDestroy(ctx->graph_out);
  if (ctx->upload_done) (void)hipEventDestroy(ctx->upload_done);
  for (DevBuf* b : {&ctx->h, &ctx->qkv, &ctx->attn, &ctx->x1, &ctx->h2, &ctx->a, &ctx->meta_dev, &ctx->part_o,
                    &ctx->part_ml, &ctx->gemm_ws, &ctx->graph_meta, &ctx->moe_idx, &ctx->moe_out, &ctx->kv_stage,
                    &ctx->kv_items})
    if (b->p) (void)hipFree(b->p);
  if (ctx->meta_host) (void)hipHostFree(ctx->meta_host);
  if (ctx->kv_host) (void)hipHostFree(ctx->kv_host);
  if (ctx->kv_upload_done) (void)hipEventDestroy(ctx->kv_upload_done);
  delete ctx;
}

extern "C" const char* nf_last_error(const nf_ctx* ctx) { return ctx ? ctx->err.c_str() : "null context"; }

namespace {

bool weights_ok(const nf_layer_cfg& c, const nf_layer_weights& w) {
  return w.g_attn && w.w_qkv && w.w_o && w.g_ffn && w.w_gate_up && w.w_down && (c.n_experts == 0 || w.w_router);
}

// Stack call: validate the layer arrays (host checks only).
nf_status check_stack_args(nf_ctx* ctx, const nf_layer_cfg* cfg, int32_t n_layers, const nf_layer_weights* w,
                           const nf_kv_pool* pools, int32_t flags) {
  if (n_layers < 1 || !w || !pools || (flags & ~(NF_STACK_PIPELINE | NF_STACK_GRAPH))) {
    ctx->err = "nf_stack_forward: n_layers >= 1, weight and pool arrays and known flags needed";
    return NF_E_ARG;
  }
  const size_t pool_bytes =
      (size_t)pools[0].num_blocks * cfg->n_kv_heads * cfg->block_size * cfg->head_dim * sizeof(uint16_t);
  std::vector<std::pair<uintptr_t, uintptr_t>> spans;
  for (int32_t l = 0; l < n_layers; ++l) {
    if (!weights_ok(*cfg, w[l]) || !pools[l].k || !pools[l].v) {
      ctx->err = "nf_stack_forward: null weight or pool pointer in layer " + std::to_string(l);
      return NF_E_ARG;
    }
    if (pools[l].num_blocks != pools[0].num_blocks) {
      ctx->err = "nf_stack_forward: every layer's pool needs the same num_blocks";
      return NF_E_ARG;
    }
    for (const void* p : {pools[l].k, pools[l].v})
      spans.push_back({reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + pool_bytes});
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) {
      ctx->err = "nf_stack_forward: KV pools of different layers overlap";
      return NF_E_ARG;
    }
  return NF_OK;
}

// Everything a captured stack bakes into its kernel arguments, besides the metadata bytes.
std::vector<uint64_t> graph_key(const nf_ctx* ctx, const nf_layer_cfg& cfg, const StackArgs& S, const nf_plan* plan,
                                int32_t flags, const nf_batch_desc& b) {
  std::vector<uint64_t> k;
  auto u = [&](uint64_t v) { k.push_back(v); };
  auto p = [&](const void* v) { k.push_back(reinterpret_cast<uintptr_t>(v)); };
  u(ctx->ws_gen);
  u((uint64_t)flags);
  u((uint64_t)S.n_layers);
  u(((uint64_t)(uint32_t)cfg.hidden << 32) | (uint32_t)cfg.ffn);
  u(((uint64_t)(uint32_t)cfg.n_q_heads << 32) | (uint32_t)cfg.n_kv_heads);
  u(((uint64_t)(uint32_t)cfg.head_dim << 32) | (uint32_t)cfg.block_size);
  uint32_t eps, base;
  memcpy(&eps, &cfg.rms_eps, 4);
  memcpy(&base, &cfg.rope_base, 4);
  u(((uint64_t)eps << 32) | base);
  p(S.x_in);
  p(S.y);
  u((uint64_t)S.max_blocks);
  u((uint64_t)S.decode_grid);
  p(b.block_table_dev);
  u(((uint64_t)(uint32_t)b.n_decode << 32) | (uint32_t)b.n_prefill);
  for (int32_t l = 0; l < S.n_layers; ++l) {
    const nf_layer_weights& w = S.w[l];
    for (const void* q : {w.g_attn, w.w_qkv, w.w_o, w.g_ffn, w.w_gate_up, w.w_down}) p(q);
    p(S.pools[l].k);
    p(S.pools[l].v);
    u((uint64_t)S.pools[l].num_blocks);
  }
  u((uint64_t)ctx->decode_split);
  u((uint64_t)ctx->decode_nbuf);
  u((uint64_t)ctx->decode_ring);
  for (auto& row : ctx->gemm_variant) u(((uint64_t)(uint32_t)row[0] << 32) | (uint32_t)row[1]);
  if (plan) {
    u((uint64_t)plan->n_nano);
    for (int32_t j = 0; j <= plan->n_nano; ++j) u((uint64_t)(uint32_t)plan->bounds[j]);
    u((uint64_t)plan->n_streams);
    u((uint64_t)plan->n_ops);
    for (int32_t i = 0; i < plan->n_ops; ++i)
      u(((uint64_t)(uint32_t)plan->op_kind[i] << 40) | ((uint64_t)(uint32_t)plan->op_nano[i] << 20) |
        (uint32_t)plan->op_stream[i]);
    u((uint64_t)(uint32_t)plan->decode_max_workgroups);
    for (int32_t i = 0; plan->op_lane && i < plan->n_ops; ++i) u((uint64_t)(uint32_t)plan->op_lane[i]);
  } else {
    u(~0ull);
  }
  return k;
}

}  // namespace

// One call of the layer stack (nf_layer_forward is the one-layer, unpipelined case).
static nf_status stack_forward(nf_ctx* ctx, const nf_layer_cfg* cfg, int32_t n_layers, const nf_layer_weights* w,
                               const void* x_in, void* y_out, const nf_batch_desc* batch, nf_kv_pool* pools,
                               const nf_plan* plan, int32_t flags, hipStream_t caller) {
  BatchLayout L;
  PlanGraph g;
  Meta M;
  nf_status st = prepare_host(ctx, cfg, batch, pools[0].num_blocks, plan, L, g, M);
  if (st != NF_OK) return st;
  const bool graph = (flags & NF_STACK_GRAPH) != 0;
  if (graph && !kGraphReplayEnabled) {
    ctx->err = "captured-graph replay of the layer stack is switched off in this build";
    return NF_E_UNSUPPORTED;
  }
  if (graph && plan && plan->cu_masks) {
    ctx->err = "a captured stack cannot keep the CU masks of the plan's streams";
    return NF_E_UNSUPPORTED;
  }
  StackGraph sg;
  if ((st = build_stack_graph(g, n_layers, (flags & NF_STACK_PIPELINE) != 0, sg, ctx->err)) != NF_OK) return st;
  std::vector<hipStream_t> ss;
  if ((st = plan_resources(ctx, plan, g, sg.order.size(), ss)) != NF_OK) return st;
  StackArgs S{cfg,
              n_layers,
              w,
              static_cast<const bf16*>(x_in),
              static_cast<bf16*>(y_out),
              pools,
              batch->max_blocks,
              (plan && plan->decode_max_workgroups > 0) ? plan->decode_max_workgroups : ctx->decode_grid};
  if (!graph) {
    if ((st = upload_meta(ctx, *cfg, *batch, L, M, caller)) != NF_OK) return st;
    if (L.T == 0) return NF_OK;
    return enqueue_stack(ctx, S, g, sg, M, ss, caller);
  }
  // captured stack: replayed while its key and metadata bytes are unchanged
  MetaPack P;
  if ((st = pack_meta(ctx, *cfg, *batch, L, M, P)) != NF_OK) return st;
  if (L.T == 0) return NF_OK;
  if (!ctx->cap_stream) NF_HIP(ctx, hipStreamCreateWithFlags(&ctx->cap_stream, hipStreamNonBlocking));
  if (!ctx->graph_in) NF_HIP(ctx, hipEventCreateWithFlags(&ctx->graph_in, hipEventDisableTiming));
  if (!ctx->graph_out) NF_HIP(ctx, hipEventCreateWithFlags(&ctx->graph_out, hipEventDisableTiming));
  if (ctx->graph_meta.cap < P.total && (st = ensure(ctx, ctx->graph_meta, P.total)) != NF_OK) return st;
  std::vector<uint64_t> key = graph_key(ctx, *cfg, S, plan, flags, *batch);
  const unsigned char* staged = static_cast<const unsigned char*>(ctx->meta_host);
  const bool reuse = ctx->graph_exec && key == ctx->graph_key && ctx->graph_meta_bytes.size() == P.total &&
                     memcmp(ctx->graph_meta_bytes.data(), staged, P.total) == 0;
  if (!reuse) {
    if (ctx->graph_exec) {
      NF_HIP(ctx, hipStreamSynchronize(ctx->cap_stream));  // the last replay is done with it
      NF_HIP(ctx, hipGraphExecDestroy(ctx->graph_exec));
      ctx->graph_exec = nullptr;
    }
    if (ctx->graph) {
      NF_HIP(ctx, hipGraphDestroy(ctx->graph));
      ctx->graph = nullptr;
    }
    ctx->graph_key.clear();
    ctx->graph_meta_bytes.clear();
    if ((st = copy_meta(ctx, P, ctx->graph_meta, caller)) != NF_OK) return st;
    point_meta(P, ctx->graph_meta.p, *batch, M);
    const uint32_t timing = ctx->timing_mask;
    ctx->timing_mask = 0;
    NF_HIP(ctx, hipStreamBeginCapture(ctx->cap_stream, hipStreamCaptureModeThreadLocal));
    st = enqueue_stack(ctx, S, g, sg, M, ss, ctx->cap_stream);
    hipGraph_t gr = nullptr;
    const hipError_t e = hipStreamEndCapture(ctx->cap_stream, &gr);
    ctx->timing_mask = timing;
    if (st != NF_OK) {
      if (gr) (void)hipGraphDestroy(gr);
      return st;
    }
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamEndCapture");
    ctx->graph = gr;
    NF_HIP(ctx, hipGraphInstantiate(&ctx->graph_exec, gr, nullptr, nullptr, 0));
    ctx->graph_key = std::move(key);
    ctx->graph_meta_bytes.assign(staged, staged + P.total);
    ++ctx->graph_captures;
  }
  ++ctx->graph_launches;
  NF_HIP(ctx, hipEventRecord(ctx->graph_in, caller));
  NF_HIP(ctx, hipStreamWaitEvent(ctx->cap_stream, ctx->graph_in, 0));
  NF_HIP(ctx, hipGraphLaunch(ctx->graph_exec, ctx->cap_stream));
  NF_HIP(ctx, hipEventRecord(ctx->graph_out, ctx->cap_stream));
  NF_HIP(ctx, hipStreamWaitEvent(caller, ctx->graph_out, 0));
  return NF_OK;
}

extern "C" nf_status nf_layer_forward(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_layer_weights* w,
                                      const void* x_in, void* y_out, const nf_batch_desc* batch, nf_kv_pool* pool,
                                      const nf_plan* plan, void* stream_) {
  if (!ctx) return NF_E_ARG;
  if (!cfg || !w || !x_in || !y_out || !batch || !pool || !pool->k || !pool->v || !weights_ok(*cfg, *w)) {
    ctx->err = "null argument";
    return NF_E_ARG;
  }
  return stack_forward(ctx, cfg, 1, w, x_in, y_out, batch, pool, plan, 0, static_cast<hipStream_t>(stream_));
}

extern "C" nf_status nf_stack_forward(nf_ctx* ctx, const nf_layer_cfg* cfg, int32_t n_layers,
                                      const nf_layer_weights* weights, const void* x_in, void* y_out,
                                      const nf_batch_desc* batch, nf_kv_pool* pools, const nf_plan* plan,
                                      int32_t flags, void* stream_) {
  if (!ctx) return NF_E_ARG;
  if (!cfg || !x_in || !y_out || !batch) {
    ctx->err = "null argument";
    return NF_E_ARG;
  }
  nf_status st = check_cfg(*cfg, ctx->err);
  if (st != NF_OK) return st;
  if ((st = check_stack_args(ctx, cfg, n_layers, weights, pools, flags)) != NF_OK) return st;
  return stack_forward(ctx, cfg, n_layers, weights, x_in, y_out, batch, pools, plan, flags,
                       static_cast<hipStream_t>(stream_));
}

extern "C" nf_status nf_debug_buffer(nf_ctx* ctx, int32_t which, void** ptr, size_t* bytes) {
  if (!ctx || !ptr) return NF_E_ARG;
  DevBuf* b = nullptr;
  switch (which) {
    case 0: b = &ctx->h; break;
    case 1: b = &ctx->qkv; break;
    case 2: b = &ctx->attn; break;
    case 3: b = &ctx->x1; break;
    case 4: b = &ctx->h2; break;
    case 5: b = &ctx->a; break;
    default: ctx->err = "unknown debug buffer"; return NF_E_ARG;
  }
  *ptr = b->p;
  if (bytes) *bytes = b->cap;
  return NF_OK;
}

extern "C" nf_status nf_gemm_variants(int32_t* count, int32_t index, int32_t* out5) {
  if (count) *count = gemm_variant_count();
  if (out5) {
    if (index < 0 || index >= gemm_variant_count()) return NF_E_ARG;
    const GemmVariant v = gemm_variant(index);
    out5[0] = v.bm;
    out5[1] = v.bn;
    out5[2] = v.bk;
    out5[3] = v.ks;
    out5[4] = v.waves;
  }
  return NF_OK;
}

extern "C" nf_status nf_gemm_choice(int32_t m, int32_t n, int32_t k, int32_t epilogue, int32_t* variant,
                                    int32_t* supported) {
  if (!variant || !supported || m < 0 || n <= 0 || k <= 0 || epilogue < 0 || epilogue > 2) return NF_E_ARG;
  if (n % 8 || k % 8) return NF_E_UNSUPPORTED;
  *variant = gemm_default_variant(m, n, k, epilogue);
  *supported = gemm_variant_supported(*variant, m, n, k, epilogue) ? 1 : 0;
  return NF_OK;
}

extern "C" nf_status nf_op_gemm(nf_ctx* ctx, const void* A, const void* B, void* C, const void* R, int32_t m, int32_t n,
                                int32_t k, int32_t epilogue, int32_t variant, void* stream) {
  if (!ctx) return NF_E_ARG;
  if (!A || !B || !C || m < 0 || n <= 0 || k <= 0 || epilogue < 0 || epilogue > 2 || (epilogue == 1 && !R)) {
    ctx->err = "nf_op_gemm: bad argument";
    return NF_E_ARG;
  }
  if (n % 8 || k % 8) {
    ctx->err = "nf_op_gemm: n and k must be multiples of 8";
    return NF_E_UNSUPPORTED;
  }
  if (variant >= 0 && !gemm_variant_supported(variant, m, n, k, epilogue)) {
    ctx->err = "nf_op_gemm: variant not available for this epilogue / k";
    return NF_E_ARG;
  }
  const int v = variant < 0 ? gemm_default_variant(m, n, k, epilogue) : variant;
  const size_t wsb = gemm_workspace_bytes(v, m, n);
  if (wsb) {
    nf_status st = ensure(ctx, ctx->gemm_ws, wsb);
    if (st != NF_OK) return st;
  }
  NF_HIP(ctx, launch_gemm(static_cast<const bf16*>(A), static_cast<const bf16*>(B), static_cast<bf16*>(C),
                          static_cast<const bf16*>(R), m, n, k, epilogue, v, static_cast<hipStream_t>(stream),
                          static_cast<float*>(ctx->gemm_ws.p), ctx->gemm_ws.cap));
  return NF_OK;
}

extern "C" nf_status nf_op_gemm_noalloc(nf_ctx* ctx, const void* A, const void* B, void* C, const void* R, int32_t m,
                                        int32_t n, int32_t k, int32_t epilogue, int32_t variant, void* stream) {
  if (!ctx) return NF_E_ARG;
  if (!A || !B || !C || m < 0 || n <= 0 || k <= 0 || epilogue < 0 || epilogue > 2 || (epilogue == 1 && !R)) {
    ctx->err = "nf_op_gemm_noalloc: bad argument";
    return NF_E_ARG;
  }
  if (n % 8 || k % 8) {
    ctx->err = "nf_op_gemm_noalloc: n and k must be multiples of 8";
    return NF_E_UNSUPPORTED;
  }
  if (variant >= 0 && !gemm_variant_supported(variant, m, n, k, epilogue)) {
    ctx->err = "nf_op_gemm_noalloc: variant not available for this epilogue / k";
    return NF_E_ARG;
  }
  const int v = variant < 0 ? gemm_default_variant(m, n, k, epilogue) : variant;
  if (gemm_workspace_bytes(v, m, n) > kNoAllocScratchBytes) {
    ctx->err = "nf_op_gemm_noalloc: the split-K partials of this product exceed the 64 MiB static scratch";
    return NF_E_CAPACITY;
  }
  NF_HIP(ctx, launch_gemm(static_cast<const bf16*>(A), static_cast<const bf16*>(B), static_cast<bf16*>(C),
                          static_cast<const bf16*>(R), m, n, k, epilogue, v, static_cast<hipStream_t>(stream),
                          static_cast<float*>(ctx->scratch), kNoAllocScratchBytes));
  return NF_OK;
}

extern "C" nf_status nf_op_rmsnorm(nf_ctx* ctx, const void* x, const void* g, void* out, int32_t m, int32_t n, float eps,
                                   void* stream) {
  if (!ctx) return NF_E_ARG;
  if (!x || !g || !out || m < 0 || n <= 0 || n % 8 || !(eps >= 0.0f)) {
    ctx->err = "nf_op_rmsnorm: bad argument (n must be a positive multiple of 8)";
    return NF_E_ARG;
  }
  NF_HIP(ctx, launch_rmsnorm(static_cast<const bf16*>(x), static_cast<const bf16*>(g), static_cast<bf16*>(out), m, n,
                             eps, static_cast<hipStream_t>(stream)));
  return NF_OK;
}

extern "C" nf_status nf_op_rope_kv_append(nf_ctx* ctx, const nf_layer_cfg* cfg, void* qkv, const nf_batch_desc* batch,
                                          nf_kv_pool* pool, void* stream) {
  if (!ctx) return NF_E_ARG;
  if (!cfg || !qkv || !batch || !pool || !pool->k || !pool->v) {
    ctx->err = "null argument";
    return NF_E_ARG;
  }
  BatchLayout L;
  PlanGraph g;
  Meta M;
  nf_status st = prepare_batch(ctx, cfg, batch, pool->num_blocks, nullptr, L, g, M, static_cast<hipStream_t>(stream));
  if (st != NF_OK) return st;
  NF_HIP(ctx, launch_rope_kv(static_cast<bf16*>(qkv), M.d_pos, M.d_slot, M.d_inv_freq, static_cast<bf16*>(pool->k),
                             static_cast<bf16*>(pool->v), 0, L.T, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim,
                             static_cast<hipStream_t>(stream)));
  return NF_OK;
}

// Attention of the batch's decode requests (decode) or prefill chunks, alone on `stream`.
static nf_status op_attention(nf_ctx* ctx, const char* name, const nf_layer_cfg* cfg, const void* qkv,
                              const nf_batch_desc* batch, const nf_kv_pool* pool, void* out, bool decode,
                              int32_t kv_split_blocks, void* stream) {
  if (!ctx) return NF_E_ARG;
  if (!cfg || !qkv || !batch || !pool || !pool->k || !pool->v || !out || kv_split_blocks < 0 ||
      kv_split_blocks > kMaxSplit) {
    ctx->err = std::string(name) + ": bad argument (null pointer, or kv_split_blocks outside 0..4096)";
    return NF_E_ARG;
  }
  const int saved = ctx->decode_split;
  if (kv_split_blocks > 0) ctx->decode_split = kv_split_blocks;
  BatchLayout L;
  PlanGraph g;
  Meta M;
  hipStream_t s = static_cast<hipStream_t>(stream);
  nf_status st = prepare_batch(ctx, cfg, batch, pool->num_blocks, nullptr, L, g, M, s);
  ctx->decode_split = saved;
  if (st != NF_OK) return st;
  const int nq = cfg->n_q_heads, nkv = cfg->n_kv_heads, d = cfg->head_dim;
  if (decode) {
    NF_HIP(ctx, launch_decode_attn(static_cast<const bf16*>(qkv), static_cast<const bf16*>(pool->k),
                                   static_cast<const bf16*>(pool->v), M.d_bt, batch->max_blocks, M.d_dec,
                                   (int)M.dec.size(), static_cast<float*>(ctx->part_o.p),
                                   static_cast<float*>(ctx->part_ml.p), static_cast<bf16*>(out), nq, nkv, d,
                                   ctx->decode_grid, ctx->decode_nbuf, ctx->decode_ring, s));
    NF_HIP(ctx, launch_decode_combine(M.d_comb, (int)M.comb.size(), static_cast<const float*>(ctx->part_o.p),
                                      static_cast<const float*>(ctx->part_ml.p), static_cast<bf16*>(out), nq, nkv, d,
                                      s));
  } else {
    NF_HIP(ctx, launch_prefill_attn(static_cast<const bf16*>(qkv), static_cast<const bf16*>(pool->k),
                                    static_cast<const bf16*>(pool->v), M.d_bt, batch->max_blocks, M.d_pf,
                                    (int)M.pf.size(), M.d_pcomb, (int)M.pcomb.size(),
                                    static_cast<float*>(ctx->part_o.p), static_cast<float*>(ctx->part_ml.p),
                                    static_cast<bf16*>(out), nq, nkv, d, s));
  }
  return NF_OK;
}

extern "C" nf_status nf_op_decode_attn(nf_ctx* ctx, const nf_layer_cfg* cfg, const void* qkv,
                                       const nf_batch_desc* batch, const nf_kv_pool* pool, void* out,
                                       int32_t kv_split_blocks, void* stream) {
  return op_attention(ctx, "nf_op_decode_attn", cfg, qkv, batch, pool, out, true, kv_split_blocks, stream);
}

extern "C" nf_status nf_op_prefill_attn(nf_ctx* ctx, const nf_layer_cfg* cfg, const void* qkv,
                                        const nf_batch_desc* batch, const nf_kv_pool* pool, void* out, void* stream) {
  return op_attention(ctx, "nf_op_prefill_attn", cfg, qkv, batch, pool, out, false, 0, stream);
}

extern "C" nf_status nf_op_moe_ffn(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_layer_weights* w, const void* h2,
                                   const void* x1, void* y, int32_t n_tokens, int32_t* sel_out, float* wts_out,
                                   void* stream) {
  if (!ctx) return NF_E_ARG;
  if (!cfg || !w || !h2 || !x1 || !y || n_tokens < 0 || !w->w_gate_up || !w->w_down || !w->w_router) {
    ctx->err = "nf_op_moe_ffn: bad argument";
    return NF_E_ARG;
  }
  nf_status st = check_cfg(*cfg, ctx->err);
  if (st != NF_OK) return st;
  if (cfg->n_experts == 0) {
    ctx->err = "nf_op_moe_ffn: the layer shape has a dense FFN";
    return NF_E_UNSUPPORTED;
  }
  if (n_tokens == 0) return NF_OK;
  if ((st = ensure_workspace(ctx, *cfg, n_tokens)) != NF_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const MoeIdx ix = moe_idx(ctx);
  if ((st = moe_ffn_rows(ctx, *cfg, *w, static_cast<const bf16*>(h2), static_cast<const bf16*>(x1),
                         static_cast<bf16*>(y), 0, n_tokens, ix.grp, s)) != NF_OK)
    return st;
  const size_t n = (size_t)2 * n_tokens;
  if (sel_out) NF_HIP(ctx, hipMemcpyAsync(sel_out, ix.sel, n * 4, hipMemcpyDeviceToDevice, s));
  if (wts_out) NF_HIP(ctx, hipMemcpyAsync(wts_out, ix.wts, n * 4, hipMemcpyDeviceToDevice, s));
  return NF_OK;
}

// KV offload / reload: validate on the host, upload the move items, then gather + copy out
// or copy in + scatter, all on `stream`.
static nf_status kv_move(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_kv_pool* pool, const nf_kv_ranges* ranges,
                         bool reload, void* host, hipStream_t s) {
  if (!ctx) return NF_E_ARG;
  if (!cfg || !pool || !pool->k || !pool->v || !ranges || !host) {
    ctx->err = "null argument";
    return NF_E_ARG;
  }
  nf_status st = check_cfg(*cfg, ctx->err);
  if (st != NF_OK) return st;
  std::vector<KvMoveItem> items;
  int64_t n_rows = 0;
  if ((st = build_kv_moves(*cfg, *ranges, pool->num_blocks, reload, items, n_rows, ctx->err)) != NF_OK) return st;
  if (items.empty()) return NF_OK;
  const size_t row_bytes = (size_t)2 * cfg->n_kv_heads * cfg->head_dim * sizeof(uint16_t);
  const size_t bytes = (size_t)n_rows * row_bytes, item_bytes = items.size() * sizeof(KvMoveItem);
  if ((st = ensure(ctx, ctx->kv_stage, bytes)) != NF_OK) return st;
  if ((st = ensure(ctx, ctx->kv_items, item_bytes)) != NF_OK) return st;
  if (!ctx->kv_upload_done) NF_HIP(ctx, hipEventCreateWithFlags(&ctx->kv_upload_done, hipEventDisableTiming));
  if (ctx->kv_upload_pending) {
    NF_HIP(ctx, hipEventSynchronize(ctx->kv_upload_done));  // item staging free again
    ctx->kv_upload_pending = false;
  }
  if (ctx->kv_host_cap < item_bytes) {
    if (ctx->kv_host) NF_HIP(ctx, hipHostFree(ctx->kv_host));
    ctx->kv_host = nullptr;
    const size_t cap = align_up(item_bytes, 1 << 16);
    NF_HIP(ctx, hipHostMalloc(&ctx->kv_host, cap, hipHostMallocDefault));
    ctx->kv_host_cap = cap;
  }
  memcpy(ctx->kv_host, items.data(), item_bytes);
  NF_HIP(ctx, hipMemcpyAsync(ctx->kv_items.p, ctx->kv_host, item_bytes, hipMemcpyHostToDevice, s));
  NF_HIP(ctx, hipEventRecord(ctx->kv_upload_done, s));
  ctx->kv_upload_pending = true;
  bf16* stage = static_cast<bf16*>(ctx->kv_stage.p);
  const KvMoveItem* d_items = static_cast<const KvMoveItem*>(ctx->kv_items.p);
  bf16* kp = static_cast<bf16*>(pool->k);
  bf16* vp = static_cast<bf16*>(pool->v);
  if (reload) {
    NF_HIP(ctx, hipMemcpyAsync(stage, host, bytes, hipMemcpyHostToDevice, s));
    NF_HIP(ctx, launch_kv_move(true, kp, vp, stage, d_items, (int)items.size(), cfg->n_kv_heads, cfg->head_dim, s));
  } else {
    NF_HIP(ctx, launch_kv_move(false, kp, vp, stage, d_items, (int)items.size(), cfg->n_kv_heads, cfg->head_dim, s));
    NF_HIP(ctx, hipMemcpyAsync(host, stage, bytes, hipMemcpyDeviceToHost, s));
  }
  return NF_OK;
}

extern "C" nf_status nf_kv_offload(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_kv_pool* pool,
                                   const nf_kv_ranges* ranges, void* host_dst, void* stream) {
  return kv_move(ctx, cfg, pool, ranges, false, host_dst, static_cast<hipStream_t>(stream));
}

extern "C" nf_status nf_kv_reload(nf_ctx* ctx, const nf_layer_cfg* cfg, nf_kv_pool* pool, const nf_kv_ranges* ranges,
                                  const void* host_src, void* stream) {
  return kv_move(ctx, cfg, pool, ranges, true, const_cast<void*>(host_src), static_cast<hipStream_t>(stream));
}

extern "C" nf_status nf_ctx_set_timing(nf_ctx* ctx, uint32_t class_mask) {
  if (!ctx) return NF_E_ARG;
  ctx->timing_mask = class_mask;
  ctx->timed.clear();
  ctx->timing_pool_used = 0;
  return NF_OK;
}

extern "C" nf_status nf_timing_summary(nf_ctx* ctx, int32_t cls, int32_t* count, double* total_ms, double* min_ms,
                                       double* max_ms) {
  if (!ctx || cls < 0 || cls >= NF_K_CLASSES || !count || !total_ms) return NF_E_ARG;
  int32_t n = 0;
  double tot = 0.0, mn = 1e300, mx = 0.0;
  for (auto& t : ctx->timed) {
    if (t.cls != cls) continue;
    NF_HIP(ctx, hipEventSynchronize(t.stop));
    float ms = 0.0f;
    NF_HIP(ctx, hipEventElapsedTime(&ms, t.start, t.stop));
    ++n;
    tot += ms;
    mn = std::min(mn, (double)ms);
    mx = std::max(mx, (double)ms);
  }
  *count = n;
  *total_ms = tot;
  if (min_ms) *min_ms = n ? mn : 0.0;
  if (max_ms) *max_ms = n ? mx : 0.0;
  return NF_OK;
}

// Internal knobs used by the profiler (not in the public header).
extern "C" nf_status nf_ctx_set_decode_split(nf_ctx* ctx, int32_t blocks) {
  if (!ctx || blocks < 0 || blocks > kMaxSplit) return NF_E_ARG;
  ctx->decode_split = blocks;
  return NF_OK;
}
extern "C" nf_status nf_ctx_set_prefill_chunk(nf_ctx* ctx, int32_t keys) {
  if (!ctx || keys < 0 || keys > kPrefillMaxChunkKeys || keys % 32) return NF_E_ARG;
  ctx->prefill_chunk = keys;
  return NF_OK;
}
extern "C" nf_status nf_ctx_set_decode_launch(nf_ctx* ctx, int32_t max_workgroups, int32_t nbuf, int32_t ring) {
  if (!ctx || max_workgroups < 0 || !decode_config_supported(nbuf, ring)) return NF_E_ARG;
  ctx->decode_grid = max_workgroups;
  ctx->decode_nbuf = nbuf;
  ctx->decode_ring = ring;
  return NF_OK;
}
extern "C" nf_status nf_ctx_graph_stats(nf_ctx* ctx, int64_t* captures, int64_t* launches) {
  if (!ctx || !captures || !launches) return NF_E_ARG;
  *captures = ctx->graph_captures;
  *launches = ctx->graph_launches;
  return NF_OK;
}
extern "C" nf_status nf_ctx_set_gemm_variant(nf_ctx* ctx, int32_t kind, int32_t which, int32_t variant) {
  if (!ctx || kind < 0 || kind >= NF_OP_KINDS || which < 0 || which > 1 || variant < -1 ||
      variant >= gemm_variant_count())
    return NF_E_ARG;
  ctx->gemm_variant[kind][which] = variant;
  return NF_OK;
}
