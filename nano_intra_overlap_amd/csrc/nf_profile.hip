// Offline profilers (NanoFlow summary page, "Kernel Profiling and Interference Modeling";
// slides "Profiling interference" and "Modeling interference").
//
// nf_profile_ops — interference-free profiling: every nano-operation kind at every batch
// size step, 2 step, ..., max_tokens (the pages use multiples of 128 up to the dense batch),
// each kernel timed in every implementation the library has (GEMM tile configurations,
// decode split-KV chunk sizes and blocks per softmax step), keeping the best: D_best.
//
// nf_profile_interference — pairwise interference between the compute class (an
// Up/Gate/Down nano-op) and the memory class (decode attention): for each resource split
// the two run concurrently on their own streams and each one's speed is recorded relative
// to its own interference-free best (P). On this GPU the resource split is physical: a CU
// mask per stream (R = share of CUs given to the memory stream, the GEMM keeps the rest),
// or a shared GPU with the memory op's workgroup count bounded.
//
// Both use synthetic data filled on the device and the same kernels as nf_layer_forward.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <functional>
#include <sstream>

#include "nf_internal.h"
#include "nf_json.h"

using namespace nf;

namespace {

__global__ void fill_kernel(bf16* p, size_t n, uint32_t seed, float scale) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint32_t h = (uint32_t)i * 0x9E3779B1u ^ seed;
    h ^= h >> 16;
    h *= 0x7FEB352Du;
    h ^= h >> 15;
    const float u = (float)(h & 0xFFFFFF) * (1.0f / 16777216.0f);  // [0, 1)
    p[i] = (bf16)((2.0f * u - 1.0f) * scale);
  }
}

struct Buf {
  void* p = nullptr;
  size_t bytes = 0;
  ~Buf() {
    if (p) (void)hipFree(p);
  }
  hipError_t alloc(size_t b) {
    bytes = b;
    return hipMalloc(&p, std::max<size_t>(b, 256));
  }
  void free() {
    if (p) (void)hipFree(p);
    p = nullptr;
    bytes = 0;
  }
  template <class T>
  T* as() const {
    return static_cast<T*>(p);
  }
};

struct Err {
  nf_status st = NF_OK;
  std::string msg;
};

#define PF_HIP(expr)                                         \
  do {                                                       \
    hipError_t e_ = (expr);                                  \
    if (e_ != hipSuccess) {                                  \
      E.st = NF_E_HIP;                                       \
      E.msg = std::string(#expr) + ": " + hipGetErrorString(e_); \
      return false;                                          \
    }                                                        \
  } while (0)

bool fill(Err& E, Buf& b, size_t n, uint32_t seed, float scale, hipStream_t s) {
  hipLaunchKernelGGL(fill_kernel, dim3(2048), dim3(256), 0, s, b.as<bf16>(), n, seed, scale);
  PF_HIP(hipGetLastError());
  return true;
}

// Known-size copy: 16 bytes per lane, grid-stride, nontemporal loads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ void copy_ref_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = __builtin_nontemporal_load(src + i);
}

// Average time (ms) of fn over reps runs on stream s, after one warm-up run.
bool time_ms(Err& E, hipStream_t s, int reps, const std::function<hipError_t()>& fn, double& out) {
  hipEvent_t a, b;
  PF_HIP(hipEventCreate(&a));
  PF_HIP(hipEventCreate(&b));
  bool ok = true;
  hipError_t e = fn();
  if (e == hipSuccess) e = hipEventRecord(a, s);
  for (int i = 0; i < reps && e == hipSuccess; ++i) e = fn();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (e != hipSuccess) {
    E.st = NF_E_HIP;
    E.msg = std::string("profiling launch failed: ") + hipGetErrorString(e);
    ok = false;
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  out = ms / reps;
  return ok;
}

// Synthetic decode batch: n requests with the template's contexts (cycled), each on its
// own run of physical blocks; a pool and device metadata for the decode kernels.
struct DecodeSet {
  int n = 0;
  int max_blocks = 0;
  int num_blocks = 0;
  std::vector<int32_t> ctx, bt;
  BatchLayout L;
  PlanGraph g;
  Buf d_bt, d_items, d_comb, d_part_o, d_part_ml;
  Meta M;
};

bool build_decode_set(Err& E, const nf_layer_cfg& c, const nf_batch_desc& tmpl, int n, int split, DecodeSet& D,
                      bool upload_table) {
  D.n = n;
  D.ctx.resize(n);
  int64_t need_total = 0;
  int maxb = 1;
  for (int i = 0; i < n; ++i) {
    D.ctx[i] = tmpl.n_decode > 0 ? tmpl.decode_ctx_len[i % tmpl.n_decode] : 1024;
    const int nb = (D.ctx[i] + 1 + kBlock - 1) / kBlock;
    need_total += nb;
    maxb = std::max(maxb, nb);
  }
  D.max_blocks = maxb;
  D.num_blocks = (int)need_total;
  D.bt.assign((size_t)n * maxb, -1);
  int64_t off = 0;
  for (int i = 0; i < n; ++i) {
    const int nb = (D.ctx[i] + 1 + kBlock - 1) / kBlock;
    for (int j = 0; j < nb; ++j) D.bt[(size_t)i * maxb + j] = (int32_t)(off + j);
    off += nb;
  }
  nf_batch_desc b{};
  b.n_decode = n;
  b.decode_ctx_len = D.ctx.data();
  b.block_table = D.bt.data();
  b.max_blocks = maxb;
  std::string err;
  nf_status st = build_layout(c, b, D.num_blocks, D.L, err);
  if (st == NF_OK) st = build_plan_graph(D.L, nullptr, D.g, err);
  if (st != NF_OK) {
    E.st = st;
    E.msg = err;
    return false;
  }
  build_work(D.L, D.g, split, 0, c.n_q_heads, c.n_kv_heads, D.M);
  const int G = c.n_q_heads / c.n_kv_heads;
  if (upload_table) {
    PF_HIP(D.d_bt.alloc(D.bt.size() * 4));
    PF_HIP(hipMemcpy(D.d_bt.p, D.bt.data(), D.bt.size() * 4, hipMemcpyHostToDevice));
  }
  PF_HIP(D.d_items.alloc(std::max<size_t>(1, D.M.dec.size()) * sizeof(DecodeItem)));
  if (!D.M.dec.empty())
    PF_HIP(hipMemcpy(D.d_items.p, D.M.dec.data(), D.M.dec.size() * sizeof(DecodeItem), hipMemcpyHostToDevice));
  PF_HIP(D.d_comb.alloc(std::max<size_t>(1, D.M.comb.size()) * sizeof(CombineItem)));
  if (!D.M.comb.empty())
    PF_HIP(hipMemcpy(D.d_comb.p, D.M.comb.data(), D.M.comb.size() * sizeof(CombineItem), hipMemcpyHostToDevice));
  const size_t parts = (size_t)std::max(D.M.n_parts, 1) * c.n_kv_heads * G;
  PF_HIP(D.d_part_o.alloc(parts * c.head_dim * 4));
  PF_HIP(D.d_part_ml.alloc(parts * 2 * 4));
  return true;
}

struct Scratch {
  Buf x, g, wqkv, wo, wgu, wd, h, qkv, attn, x1, h2, a, y, kpool, vpool, pos, slot, inv;
  Buf wr, moe_out, moe_idx;  // MoE: router, grouped expert outputs, index arrays
};

bool alloc_dense(Err& E, const nf_layer_cfg& c, int max_t, Scratch& S, hipStream_t s) {
  const size_t H = c.hidden, F = c.ffn, W = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim,
               Q = (size_t)c.n_q_heads * c.head_dim, T = max_t;
  const size_t E_ = c.n_experts > 0 ? (size_t)c.n_experts : 1, fan = c.n_experts > 0 ? 2 : 1;
  struct A {
    Buf* b;
    size_t n;
    float scale;
  } list[] = {{&S.x, T * H, 2.0f},      {&S.g, H, 1.0f},       {&S.wqkv, W * H, 0.03f}, {&S.wo, H * Q, 0.03f},
              {&S.wgu, E_ * 2 * F * H, 0.03f}, {&S.wd, E_ * H * F, 0.03f}, {&S.h, T * H, 1.0f}, {&S.qkv, T * W, 1.0f},
              {&S.attn, T * Q, 1.0f},    {&S.x1, T * H, 1.0f},  {&S.h2, T * H, 1.0f},    {&S.a, fan * T * F, 1.0f},
              {&S.y, T * H, 1.0f}};
  uint32_t seed = 1;
  for (auto& e : list) {
    PF_HIP(e.b->alloc(e.n * 2));
    if (!fill(E, *e.b, e.n, seed++, e.scale, s)) return false;
  }
  if (c.n_experts > 0) {
    PF_HIP(S.wr.alloc(E_ * H * 2));
    if (!fill(E, S.wr, E_ * H, seed++, 0.05f, s)) return false;
    PF_HIP(S.moe_out.alloc(2 * T * H * 2));
    PF_HIP(S.moe_idx.alloc(16 * 2 * T + 8 * E_));
  }
  // a small pool and positions / slots for the rotary + KV append kernel
  const size_t blocks = T / kBlock + 1;
  const size_t per_block = (size_t)c.n_kv_heads * kBlock * c.head_dim;
  PF_HIP(S.kpool.alloc(blocks * per_block * 2));
  PF_HIP(S.vpool.alloc(blocks * per_block * 2));
  if (!fill(E, S.kpool, blocks * per_block, seed++, 1.3f, s)) return false;
  if (!fill(E, S.vpool, blocks * per_block, seed++, 1.3f, s)) return false;
  std::vector<int32_t> pos(T), slot(T);
  for (size_t t = 0; t < T; ++t) pos[t] = slot[t] = (int32_t)t;
  std::vector<float> inv(c.head_dim / 2);
  for (int i = 0; i < c.head_dim / 2; ++i) inv[i] = (float)std::pow((double)c.rope_base, -2.0 * i / c.head_dim);
  PF_HIP(S.pos.alloc(T * 4));
  PF_HIP(S.slot.alloc(T * 4));
  PF_HIP(S.inv.alloc(inv.size() * 4));
  PF_HIP(hipMemcpy(S.pos.p, pos.data(), T * 4, hipMemcpyHostToDevice));
  PF_HIP(hipMemcpy(S.slot.p, slot.data(), T * 4, hipMemcpyHostToDevice));
  PF_HIP(hipMemcpy(S.inv.p, inv.data(), inv.size() * 4, hipMemcpyHostToDevice));
  return true;
}

// The MoE FFN of m tokens (router + dispatch, grouped Up/Gate, grouped Down, combine) on
// the scratch buffers, default grouped tiles.
hipError_t moe_ffn_op(const nf_layer_cfg& c, Scratch& S, int m, hipStream_t s) {
  const int H = c.hidden, F = c.ffn, Ex = c.n_experts, rows = 2 * m;
  char* b = static_cast<char*>(S.moe_idx.p);
  const size_t n = (size_t)2 * m;
  int32_t* sel = reinterpret_cast<int32_t*>(b);
  float* wts = reinterpret_cast<float*>(b + 4 * n);
  int32_t* pos = reinterpret_cast<int32_t*>(b + 8 * n);
  int32_t* src = reinterpret_cast<int32_t*>(b + 12 * n);
  int32_t* grp = reinterpret_cast<int32_t*>(b + 16 * n);
  hipError_t e = launch_moe_route(S.h2.as<bf16>(), S.wr.as<bf16>(), 0, m, H, Ex, sel, wts, pos, src, grp, s);
  if (e == hipSuccess)
    e = launch_gemm_grouped(S.h2.as<bf16>(), src, S.wgu.as<bf16>(), (long long)2 * F * H, S.a.as<bf16>(), grp, Ex,
                            rows, F, H, 2, gemm_grouped_default_variant(rows, Ex, H, 2), s);
  if (e == hipSuccess)
    e = launch_gemm_grouped(S.a.as<bf16>(), nullptr, S.wd.as<bf16>(), (long long)H * F, S.moe_out.as<bf16>(), grp, Ex,
                            rows, H, F, 0, gemm_grouped_default_variant(rows, Ex, F, 0), s);
  if (e == hipSuccess)
    e = launch_moe_combine(S.x1.as<bf16>(), S.moe_out.as<bf16>(), pos, wts, S.y.as<bf16>(), 0, m, H, s);
  return e;
}

// Best GEMM variant for (m, n, k, epi): returns ms and variant.
bool best_gemm(Err& E, hipStream_t s, const bf16* A, const bf16* B, bf16* C, const bf16* R, int m, int n, int k,
               int epi, int reps, double& best_ms, int& best_v) {
  best_ms = 1e30;
  best_v = -1;
  size_t wsb = 0;
  for (int v = 0; v < gemm_variant_count(); ++v)
    if (gemm_variant_supported(v, m, n, k, epi)) wsb = std::max(wsb, gemm_workspace_bytes(v, m, n));
  Buf ws;
  if (wsb) PF_HIP(ws.alloc(wsb));
  for (int v = 0; v < gemm_variant_count(); ++v) {
    if (!gemm_variant_supported(v, m, n, k, epi)) continue;
    double ms;
    if (!time_ms(E, s, reps, [&] { return launch_gemm(A, B, C, R, m, n, k, epi, v, s, ws.as<float>(), wsb); }, ms))
      return false;
    if (ms < best_ms) {
      best_ms = ms;
      best_v = v;
    }
  }
  return true;
}

std::string cfg_json(const nf_layer_cfg& c) {
  std::ostringstream o;
  o << "{\"hidden\": " << c.hidden << ", \"n_q_heads\": " << c.n_q_heads << ", \"n_kv_heads\": " << c.n_kv_heads
    << ", \"head_dim\": " << c.head_dim << ", \"ffn\": " << c.ffn << ", \"n_experts\": " << c.n_experts << "}";
  return o.str();
}

bool write_file(Err& E, const char* path, const std::string& text) {
  FILE* f = fopen(path, "w");
  if (!f) {
    E.st = NF_E_IO;
    E.msg = std::string("cannot write ") + path;
    return false;
  }
  fputs(text.c_str(), f);
  fclose(f);
  return true;
}

// Decode attention timing for one launch configuration. bt / bt_stride: the device block
// table the items index (request r's row starts at r * bt_stride).
bool time_decode(Err& E, hipStream_t s, const nf_layer_cfg& c, DecodeSet& D, const bf16* qkv, const bf16* kp,
                 const bf16* vp, const int32_t* bt, int bt_stride, bf16* out, int grid, int nb, int ring, int reps,
                 double& ms) {
  return time_ms(E, s, reps,
                 [&] {
                   hipError_t e = launch_decode_attn(qkv, kp, vp, bt, bt_stride, D.d_items.as<DecodeItem>(),
                                                     (int)D.M.dec.size(), D.d_part_o.as<float>(),
                                                     D.d_part_ml.as<float>(), out, c.n_q_heads, c.n_kv_heads,
                                                     c.head_dim, grid, nb, ring, s);
                   if (e != hipSuccess) return e;
                   return launch_decode_combine(D.d_comb.as<CombineItem>(), (int)D.M.comb.size(),
                                                D.d_part_o.as<float>(), D.d_part_ml.as<float>(), out, c.n_q_heads,
                                                c.n_kv_heads, c.head_dim, s);
                 },
                 ms);
}

}  // namespace

// ---------------------------------------------------------------------------------------

extern "C" nf_status nf_profile_ops(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_batch_desc* tmpl,
                                    int32_t num_blocks, int32_t step, int32_t max_tokens, const char* out_json) {
  if (!ctx || !cfg || !tmpl || !out_json || step < 1 || max_tokens < step || max_tokens > 65536) return NF_E_ARG;
  (void)num_blocks;
  std::string err;
  nf_status st = check_cfg(*cfg, err);
  if (st != NF_OK) return st;
  Err E;
  const nf_layer_cfg& c = *cfg;
  hipStream_t s;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return NF_E_HIP;
  std::ostringstream o;
  bool ok = [&]() -> bool {
    Scratch S;
    if (!alloc_dense(E, c, max_tokens, S, s)) return false;
    const int H = c.hidden, F = c.ffn, nq = c.n_q_heads, nkv = c.n_kv_heads, d = c.head_dim;
    const int W = (nq + 2 * nkv) * d, Q = nq * d;
    const int reps = 5;
    std::ostringstream kqv, oo, ugd, dec, pf, vk, vo, vu, vd;
    for (int m = step; m <= max_tokens; m += step) {
      double tn, tg, tr, to, tu, td;
      int v1, v2, v3;
      if (!time_ms(E, s, reps, [&] { return launch_rmsnorm(S.x.as<bf16>(), S.g.as<bf16>(), S.h.as<bf16>(), m, H,
                                                             c.rms_eps, s); }, tn))
        return false;
      if (!best_gemm(E, s, S.h.as<bf16>(), S.wqkv.as<bf16>(), S.qkv.as<bf16>(), nullptr, m, W, H, 0, reps, tg, v1))
        return false;
      if (!time_ms(E, s, reps, [&] { return launch_rope_kv(S.qkv.as<bf16>(), S.pos.as<int32_t>(),
                                                             S.slot.as<int32_t>(), S.inv.as<float>(),
                                                             S.kpool.as<bf16>(), S.vpool.as<bf16>(), 0, m, nq, nkv,
                                                             d, s); }, tr))
        return false;
      if (!best_gemm(E, s, S.attn.as<bf16>(), S.wo.as<bf16>(), S.x1.as<bf16>(), S.x.as<bf16>(), m, H, Q, 1, reps, to,
                     v2))
        return false;
      double tug, tdown = 0.0;
      int v4;
      if (c.n_experts > 0) {  // the MoE FFN as one nano-op (its tiles are chosen per call)
        if (!time_ms(E, s, reps, [&] { return moe_ffn_op(c, S, m, s); }, tug)) return false;
        v3 = gemm_grouped_default_variant(2 * m, c.n_experts, c.hidden, 2);
        v4 = gemm_grouped_default_variant(2 * m, c.n_experts, c.ffn, 0);
      } else {
        if (!best_gemm(E, s, S.h2.as<bf16>(), S.wgu.as<bf16>(), S.a.as<bf16>(), nullptr, m, F, H, 2, reps, tug, v3))
          return false;
        if (!best_gemm(E, s, S.a.as<bf16>(), S.wd.as<bf16>(), S.y.as<bf16>(), S.x1.as<bf16>(), m, H, F, 1, reps, tdown,
                       v4))
          return false;
      }
      tu = tn + tug + tdown;
      td = tn + tg + tr;
      const char* sep = m == step ? "" : ", ";
      kqv << sep << "[" << m << ", " << json::num(td) << "]";
      oo << sep << "[" << m << ", " << json::num(to) << "]";
      ugd << sep << "[" << m << ", " << json::num(tu) << "]";
      vk << sep << "[" << m << ", " << v1 << "]";
      vo << sep << "[" << m << ", " << v2 << "]";
      vu << sep << "[" << m << ", " << v3 << ", " << v4 << "]";
    }
    // decode attention: n decode tokens with the template's contexts
    {
      DecodeSet big;
      const int n_max = max_tokens;
      if (!build_decode_set(E, c, *tmpl, n_max, 32, big, true)) return false;
      const size_t per_block = (size_t)nkv * kBlock * d;
      Buf kp, vp, out;
      PF_HIP(kp.alloc((size_t)big.num_blocks * per_block * 2));
      PF_HIP(vp.alloc((size_t)big.num_blocks * per_block * 2));
      PF_HIP(out.alloc((size_t)n_max * Q * 2));
      if (!fill(E, kp, (size_t)big.num_blocks * per_block, 77, 1.3f, s)) return false;
      if (!fill(E, vp, (size_t)big.num_blocks * per_block, 78, 1.3f, s)) return false;
      bool first = true;
      for (int n = step; n <= n_max; n += step) {
        double best = 1e30;
        int bsplit = 0, bnb = 0, bring = 0;
        for (int split : {0, 16, 32, 64, 128})
          for (auto cf : {std::pair<int, int>{1, 2}, {1, 3}, {2, 2}}) {
            DecodeSet D;
            if (!build_decode_set(E, c, *tmpl, n, split, D, false)) return false;
            double ms;
            // requests 0..n-1 of D have the contexts of big's first n rows: use big's table
            if (!time_decode(E, s, c, D, S.qkv.as<bf16>(), kp.as<bf16>(), vp.as<bf16>(), big.d_bt.as<int32_t>(),
                             big.max_blocks, out.as<bf16>(), 0, cf.first, cf.second, 3, ms))
              return false;
            if (ms < best) {
              best = ms;
              bsplit = split;
              bnb = cf.first;
              bring = cf.second;
            }
          }
        dec << (first ? "" : ", ") << "[" << n << ", " << json::num(best) << ", " << bsplit << ", " << bnb << ", "
            << bring << "]";
        first = false;
      }
    }
    // prefill attention: one chunk of length len, no cached prefix (work list and key
    // chunks as the layer builds them, partials merged by the combine kernel)
    {
      const int lmax = std::min(max_tokens, 2048);
      std::vector<int32_t> bt((lmax + kBlock - 1) / kBlock);
      for (size_t i = 0; i < bt.size(); ++i) bt[i] = (int32_t)i;
      Buf d_bt, items, combs, part_o, part_ml, out;
      PF_HIP(d_bt.alloc(bt.size() * 4));
      PF_HIP(hipMemcpy(d_bt.p, bt.data(), bt.size() * 4, hipMemcpyHostToDevice));
      PF_HIP(out.alloc((size_t)lmax * Q * 2));
      bool first = true;
      for (int len = step; len <= lmax; len += step) {
        std::vector<PrefillReq> reqs{PrefillReq{0, 0, len, 0}};
        std::vector<PrefillItem> its;
        std::vector<CombineItem> cmb;
        int32_t n_parts = 0;
        build_prefill_work(reqs, nq, nkv, prefill_chunk_keys(reqs, nq, nkv), its, cmb, n_parts);
        items.free();
        combs.free();
        part_o.free();
        part_ml.free();
        PF_HIP(items.alloc(its.size() * sizeof(PrefillItem)));
        PF_HIP(hipMemcpy(items.p, its.data(), its.size() * sizeof(PrefillItem), hipMemcpyHostToDevice));
        PF_HIP(combs.alloc(std::max<size_t>(1, cmb.size()) * sizeof(CombineItem)));
        if (!cmb.empty())
          PF_HIP(hipMemcpy(combs.p, cmb.data(), cmb.size() * sizeof(CombineItem), hipMemcpyHostToDevice));
        PF_HIP(part_o.alloc((size_t)std::max(n_parts, 1) * nq * d * 4));
        PF_HIP(part_ml.alloc((size_t)std::max(n_parts, 1) * nq * 2 * 4));
        double ms;
        if (!time_ms(E, s, 3, [&] { return launch_prefill_attn(S.qkv.as<bf16>(), S.kpool.as<bf16>(),
                                                                S.vpool.as<bf16>(), d_bt.as<int32_t>(),
                                                                (int)bt.size(), items.as<PrefillItem>(),
                                                                (int)its.size(), combs.as<CombineItem>(),
                                                                (int)cmb.size(), part_o.as<float>(),
                                                                part_ml.as<float>(), out.as<bf16>(), nq, nkv, d, s); },
                     ms))
          return false;
        pf << (first ? "" : ", ") << "[" << len << ", " << json::num(ms) << "]";
        first = false;
      }
    }
    hipDeviceProp_t p;
    PF_HIP(hipGetDeviceProperties(&p, 0));
    o << "{\"device\": " << json::quote(p.gcnArchName) << ", \"cu\": " << p.multiProcessorCount
      << ", \"cfg\": " << cfg_json(c) << ", \"step\": " << step << ",\n \"ops\": {\"KQV\": [" << kqv.str()
      << "],\n  \"O\": [" << oo.str() << "],\n  \"UGD\": [" << ugd.str() << "],\n  \"DECATTN\": [" << dec.str()
      << "],\n  \"PFATTN\": [" << pf.str() << "]},\n \"best_variants\": {\"KQV\": [" << vk.str() << "], \"O\": ["
      << vo.str() << "], \"UGD\": [" << vu.str()
      << "]},\n \"notes\": \"ms per nano-op, best implementation per size; DECATTN rows are [decode tokens, ms, "
         "split-KV blocks, blocks per softmax step]\"}\n";
    return true;
  }();
  (void)hipStreamSynchronize(s);
  (void)hipStreamDestroy(s);
  if (!ok) return E.st;
  Err W;
  if (!write_file(W, out_json, o.str())) return W.st;
  return NF_OK;
}

extern "C" nf_status nf_profile_interference(nf_ctx* ctx, const nf_layer_cfg* cfg, const nf_batch_desc* tmpl,
                                             int32_t num_blocks, const float* r_grid, int32_t n_r,
                                             const char* out_json) {
  if (!ctx || !cfg || !tmpl || !out_json || n_r < 0 || (n_r > 0 && !r_grid) || n_r > 16) return NF_E_ARG;
  (void)num_blocks;
  for (int i = 0; i < n_r; ++i)
    if (!(r_grid[i] > 0.0f && r_grid[i] < 1.0f)) return NF_E_ARG;
  std::string err;
  nf_status st = check_cfg(*cfg, err);
  if (st != NF_OK) return st;
  Err E;
  const nf_layer_cfg& c = *cfg;
  const int T = tmpl->n_decode + [&] {
    int t = 0;
    for (int j = 0; j < tmpl->n_prefill; ++j) t += tmpl->prefill_len[j];
    return t;
  }();
  const int m = std::max(128, (T / 2 + 127) / 128 * 128);  // a half dense batch of rows
  const int n_dec = std::max(1, tmpl->n_decode / 2);        // the decode requests of half a batch
  std::ostringstream o;
  std::vector<hipStream_t> made;
  bool ok = [&]() -> bool {
    hipStream_t s0, s1;
    PF_HIP(hipStreamCreateWithFlags(&s0, hipStreamNonBlocking));
    made.push_back(s0);
    PF_HIP(hipStreamCreateWithFlags(&s1, hipStreamNonBlocking));
    made.push_back(s1);
    Scratch S;
    if (!alloc_dense(E, c, m, S, s0)) return false;
    const int H = c.hidden, F = c.ffn, nkv = c.n_kv_heads, d = c.head_dim, Q = c.n_q_heads * d;
    DecodeSet D;
    if (!build_decode_set(E, c, *tmpl, n_dec, 32, D, true)) return false;
    const size_t per_block = (size_t)nkv * kBlock * d;
    Buf kp, vp, out;
    PF_HIP(kp.alloc((size_t)D.num_blocks * per_block * 2));
    PF_HIP(vp.alloc((size_t)D.num_blocks * per_block * 2));
    PF_HIP(out.alloc((size_t)n_dec * Q * 2 + 256));
    if (!fill(E, kp, (size_t)D.num_blocks * per_block, 91, 1.3f, s0)) return false;
    if (!fill(E, vp, (size_t)D.num_blocks * per_block, 92, 1.3f, s0)) return false;
    PF_HIP(hipStreamSynchronize(s0));
    const int W = (c.n_q_heads + 2 * nkv) * d;
    const int vug = gemm_default_variant(m, F, H, 2), vdn = gemm_default_variant(m, H, F, 1);
    const int vqkv = gemm_default_variant(m, W, H, 0), vo = gemm_default_variant(m, H, Q, 1);
    const size_t wsb = std::max(std::max(gemm_workspace_bytes(vug, m, F), gemm_workspace_bytes(vdn, m, H)),
                                std::max(gemm_workspace_bytes(vqkv, m, W), gemm_workspace_bytes(vo, m, H)));
    Buf gws;
    if (wsb) PF_HIP(gws.alloc(wsb));
    // compute ops: one nano-op of each compute kind (the main entry is Up/Gate/Down); memory
    // op: one decode attention nano-op. The KQV product writes into the FFN activation
    // buffer, not into the qkv rows the attention reads.
    auto ugd_op = [&](hipStream_t s) -> hipError_t {
      if (c.n_experts > 0) return moe_ffn_op(c, S, m, s);
      hipError_t e = launch_gemm(S.h2.as<bf16>(), S.wgu.as<bf16>(), S.a.as<bf16>(), nullptr, m, F, H, 2, vug, s,
                                 gws.as<float>(), wsb);
      if (e != hipSuccess) return e;
      return launch_gemm(S.a.as<bf16>(), S.wd.as<bf16>(), S.y.as<bf16>(), S.x1.as<bf16>(), m, H, F, 1, vdn, s,
                         gws.as<float>(), wsb);
    };
    auto kqv_op = [&](hipStream_t s) -> hipError_t {
      return launch_gemm(S.h.as<bf16>(), S.wqkv.as<bf16>(), S.a.as<bf16>(), nullptr, m, W, H, 0, vqkv, s,
                         gws.as<float>(), wsb);
    };
    auto o_op = [&](hipStream_t s) -> hipError_t {
      return launch_gemm(S.attn.as<bf16>(), S.wo.as<bf16>(), S.y.as<bf16>(), S.x.as<bf16>(), m, H, Q, 1, vo, s,
                         gws.as<float>(), wsb);
    };
    constexpr int kMemLoops = 4;  // memory nano-ops per concurrent run
    struct Kind {
      const char* name;
      std::function<hipError_t(hipStream_t)> op;
      double best = 0.0;
    };
    std::vector<Kind> kinds = {{"UGD", ugd_op}, {"KQV", kqv_op}, {"O", o_op}};
    int grid = 0;
    auto mem_op = [&](hipStream_t s) -> hipError_t {
      hipError_t e = launch_decode_attn(S.qkv.as<bf16>(), kp.as<bf16>(), vp.as<bf16>(), D.d_bt.as<int32_t>(),
                                        D.max_blocks, D.d_items.as<DecodeItem>(), (int)D.M.dec.size(),
                                        D.d_part_o.as<float>(), D.d_part_ml.as<float>(), out.as<bf16>(),
                                        c.n_q_heads, c.n_kv_heads, d, grid, 1, 2, s);
      if (e != hipSuccess) return e;
      return launch_decode_combine(D.d_comb.as<CombineItem>(), (int)D.M.comb.size(), D.d_part_o.as<float>(),
                                   D.d_part_ml.as<float>(), out.as<bf16>(), c.n_q_heads, c.n_kv_heads, d, s);
    };
    // best times: after a warm-up (code loaded, clocks and caches settled), the fastest of
    // three rounds; every P value below is a speed relative to these
    auto best_ms = [&](const std::function<hipError_t(hipStream_t)>& op, double& best) -> bool {
      for (int i = 0; i < 10; ++i) PF_HIP(op(s0));
      best = 1e30;
      for (int r = 0; r < 3; ++r) {
        double t;
        if (!time_ms(E, s0, 5, [&] { return op(s0); }, t)) return false;
        best = std::min(best, t);
      }
      return true;
    };
    double tg_best, tm_best;
    for (Kind& k : kinds)
      if (!best_ms(k.op, k.best)) return false;
    tg_best = kinds[0].best;
    if (!best_ms(mem_op, tm_best)) return false;

    // masked entries come in pairs: the compute op on the complement of the memory mask,
    // and ("gemm_full") on the whole GPU beside the same memory mask, so a plan can give
    // each compute kind either share
    struct Cfg {
      std::string name;
      double r;
      bool masked;
      int grid;
      bool gemm_full;
    };
    std::vector<Cfg> cfgs = {{"shared", -1.0, false, 0, false}, {"shared_grid256", -1.0, false, 256, false},
                             {"shared_grid512", -1.0, false, 512, false}};
    for (int i = 0; i < n_r; ++i) {
      char nm[48];
      snprintf(nm, sizeof nm, "mask_r%.3g", r_grid[i]);
      cfgs.push_back({nm, (double)r_grid[i], true, 0, false});
      snprintf(nm, sizeof nm, "mask_r%.3g_gemm_full", r_grid[i]);
      cfgs.push_back({nm, (double)r_grid[i], true, 0, true});
    }
    o << "{\"device_cus\": 256, \"cfg\": " << cfg_json(c) << ", \"gemm_op\": \"" << (c.n_experts > 0 ? "MoE FFN (router, grouped Up/Gate+SwiGLU, grouped Down, combine), " : "Up/Gate+SwiGLU+Down, ") << m
      << " rows (KQV and O of as many rows in the *_kind fields)\", \"mem_op\": \"decode attention, " << n_dec << " requests\", \"t_gemm_best_ms\": "
      << json::num(tg_best) << ", \"t_mem_best_ms\": " << json::num(tm_best) << ",\n \"configs\": [";
    bool first = true;
    for (const Cfg& cf : cfgs) {
      uint32_t masks[2][NF_CU_MASK_WORDS];
      hipStream_t sg = s0, sm = s1;
      hipStream_t own[2] = {nullptr, nullptr};
      if (cf.masked) {
        const int per = std::min(31, std::max(1, (int)std::lround(cf.r * 32)));  // memory CUs per XCD
        for (int s = 0; s < 2; ++s)
          for (int w = 0; w < NF_CU_MASK_WORDS; ++w) masks[s][w] = 0;
        for (int i = 0; i < 256; ++i) {
          const int slot = i / 8;  // bit i -> XCD i % 8; the slot-th CU of that XCD
          masks[slot < 32 - per ? 0 : 1][i / 32] |= 1u << (i % 32);
        }
        if (cf.gemm_full) {
          for (int w = 0; w < NF_CU_MASK_WORDS; ++w) masks[0][w] = 0xFFFFFFFFu;
        } else {
          PF_HIP(hipExtStreamCreateWithCUMask(&own[0], NF_CU_MASK_WORDS, masks[0]));
          made.push_back(own[0]);
          sg = own[0];
        }
        PF_HIP(hipExtStreamCreateWithCUMask(&own[1], NF_CU_MASK_WORDS, masks[1]));
        made.push_back(own[1]);
        sm = own[1];
      }
      grid = cf.grid;
      // alone on a masked stream: slower than on the whole GPU; on the shared GPU an op
      // alone runs at its best by definition (a bounded attention grid is timed)
      double tm_alone = tm_best;
      if (cf.masked || cf.grid > 0)
        if (!time_ms(E, sm, 3, [&] { return mem_op(sm); }, tm_alone)) return false;
      const double pm_alone = std::min(1.0, tm_best / tm_alone);
      // each compute kind against the memory op: loops sized to about the same length,
      // started together; work in units of best time, the longer loop's tail ran alone
      struct Pair {
        double pg_both, pm_both, pg_alone, fg, fm;
        int lg;
      };
      std::vector<Pair> pairs;
      for (Kind& k : kinds) {
        double tg_alone = k.best;
        if (cf.masked && !cf.gemm_full)
          if (!time_ms(E, sg, 3, [&] { return k.op(sg); }, tg_alone)) return false;
        const int lm = kMemLoops;
        const int lg = std::max(1, (int)std::lround(lm * tm_alone / tg_alone));
        const double wg = lg * k.best, wm = lm * tm_best;
        const double pg_alone = std::min(1.0, k.best / tg_alone);
        // three concurrent runs; each speed is the median of its three values
        double v_pg[3], v_pm[3], v_fg[3], v_fm[3];
        for (int rep = 0; rep < 3; ++rep) {
          hipEvent_t e0, eg, em;
          PF_HIP(hipEventCreate(&e0));
          PF_HIP(hipEventCreate(&eg));
          PF_HIP(hipEventCreate(&em));
          PF_HIP(hipStreamSynchronize(sg));
          PF_HIP(hipStreamSynchronize(sm));
          PF_HIP(hipEventRecord(e0, sg));
          PF_HIP(hipStreamWaitEvent(sm, e0, 0));
          for (int i = 0; i < lg; ++i) PF_HIP(k.op(sg));
          for (int i = 0; i < lm; ++i) PF_HIP(mem_op(sm));
          PF_HIP(hipEventRecord(eg, sg));
          PF_HIP(hipEventRecord(em, sm));
          PF_HIP(hipEventSynchronize(eg));
          PF_HIP(hipEventSynchronize(em));
          float fg = 0, fm = 0;
          PF_HIP(hipEventElapsedTime(&fg, e0, eg));
          PF_HIP(hipEventElapsedTime(&fm, e0, em));
          (void)hipEventDestroy(e0);
          (void)hipEventDestroy(eg);
          (void)hipEventDestroy(em);
          const double t1 = std::min((double)fg, (double)fm);
          if (fg <= fm) {
            v_pg[rep] = wg / t1;
            v_pm[rep] = std::max(1e-3, (wm - (fm - t1) * pm_alone) / t1);
          } else {
            v_pm[rep] = wm / t1;
            v_pg[rep] = std::max(1e-3, (wg - (fg - t1) * pg_alone) / t1);
          }
          v_fg[rep] = fg;
          v_fm[rep] = fm;
        }
        auto median3 = [](double* v) {
          std::sort(v, v + 3);
          return v[1];
        };
        const double pg_both = median3(v_pg), pm_both = median3(v_pm), fg = median3(v_fg), fm = median3(v_fm);
        pairs.push_back({pg_both, pm_both, pg_alone, fg, fm, lg});
      }
      const Pair& u = pairs[0];  // Up/Gate/Down: the entry's plain fields
      const double pg_both = u.pg_both, pm_both = u.pm_both, pg_alone = u.pg_alone;
      const float fg = (float)u.fg, fm = (float)u.fm;
      const int lg = u.lg, lm = kMemLoops;
      auto kind_obj = [&](double Pair::*f) {
        std::ostringstream k;
        k << "{";
        for (size_t i = 0; i < kinds.size(); ++i)
          k << (i ? ", " : "") << json::quote(kinds[i].name) << ": " << json::num(pairs[i].*f);
        k << "}";
        return k.str();
      };
      o << (first ? "" : ",") << "\n  {\"name\": " << json::quote(cf.name) << ", \"r_mem\": " << json::num(cf.r)
        << ", \"gemm_full\": " << (cf.gemm_full ? "true" : "false")
        << ", \"decode_grid\": " << cf.grid << ", \"p_gemm_both\": " << json::num(pg_both)
        << ", \"p_mem_both\": " << json::num(pm_both) << ", \"p_gemm_alone\": " << json::num(pg_alone)
        << ", \"p_mem_alone\": " << json::num(pm_alone) << ", \"concurrent_ms\": [" << json::num(fg) << ", "
        << json::num(fm) << "], \"loops\": [" << lg << ", " << lm << "]"
        << ", \"p_gemm_both_kind\": " << kind_obj(&Pair::pg_both) << ", \"p_mem_both_kind\": " << kind_obj(&Pair::pm_both)
        << ", \"p_gemm_alone_kind\": " << kind_obj(&Pair::pg_alone);
      if (cf.masked) {
        o << ", \"cu_masks\": [";
        for (int s = 0; s < 2; ++s) {
          o << (s ? ", " : "") << "[";
          for (int w = 0; w < NF_CU_MASK_WORDS; ++w) o << (w ? ", " : "") << masks[s][w];
          o << "]";
        }
        o << "]";
      } else {
        o << ", \"cu_masks\": null";
      }
      o << "}";
      first = false;
    }
    o << "\n ]}\n";
    return true;
  }();
  for (auto s : made) {
    (void)hipStreamSynchronize(s);
    (void)hipStreamDestroy(s);
  }
  if (!ok) return E.st;
  Err W;
  if (!write_file(W, out_json, o.str())) return W.st;
  return NF_OK;
}

extern "C" nf_status nf_copy_reference(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes % 16 || reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return NF_E_ARG;
  const char* d = static_cast<const char*>(dst);
  const char* s = static_cast<const char*>(src);
  if (d < s + bytes && s < d + bytes) return NF_E_ARG;
  if (bytes == 0) return NF_OK;
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256, 8192);
  hipLaunchKernelGGL(copy_ref_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), n16);
  return hipGetLastError() == hipSuccess ? NF_OK : NF_E_HIP;
}
