// Prefill attention on gfx950 matrix cores: compute-bound, causal within each prefill chunk
// of the dense batch ("Inside nano-vLLM", prefill batching keeps request boundaries; NanoFlow
// slides, "Batch Formation"), over the paged KV pool (the chunk's own keys were appended by
// the rotary / KV-append kernel before this runs, its cached prefix is already there).
#include <type_traits>

#include "nf_internal.h"

#ifndef NF_PF_STAGES
#define NF_PF_STAGES 3
#endif

namespace nf {

// ---------------------------------------------------------------------------------------
// prefill
// ---------------------------------------------------------------------------------------
//
// A workgroup of 4 waves takes one work item — a tile of 32 x (4 / HPW) consecutive queries
// of a prefill chunk and a range of at most 1024 of the request's keys — for HPW query heads
// of one KV group: wave w handles query rows (w / HPW) * 32 .. + 31 of the tile for head
// h0 + w % HPW. The keys stream in steps of 32 through a ring of S LDS stages filled by
// direct-to-LDS loads (K and V of a step loaded once, read by every wave). Per step a wave
// computes S^T[32 keys][32 queries] = K Q^T with D/16 32x32x16 MFMAs, an online softmax per
// query (one query per lane column: its 32 keys sit in lanes l and l + 32), then
// O^T[D][32 queries] += V^T P^T with 2 D/32 MFMAs.
//
// Operand layouts, chosen so that every fragment is one 16-byte LDS read:
//  - K stage: row r = key r of the step, D dims (2 D bytes), 16-byte chunk slot p holding
//    dims 8 (p ^ fk(r)) .. + 7, fk spreading 16 consecutive rows over distinct banks.
//  - MFMA row i of S^T holds key perm32(i): the middle two quads of each 16 rows swapped,
//    which places keys 8 h .. 8 h + 7 (+16) of a query in lane half h's accumulator
//    registers 0-7 (8-15) — exactly the B operand P^T of the value product, and the value
//    fragment (A = V^T, row = dim, 8 consecutive keys) is then one chunk of a V row.
//  - V stage: row = dim, 32 keys (64 bytes), 16-byte chunk slot p holding keys
//    8 (p ^ gv(dim)) .. + 7.
// Items whose tile's keys are split over several items write fp32 partials (unnormalised
// O, running max and sum per query and head) that the decode combine kernel merges.

__device__ __forceinline__ int perm16(int i) { return (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3); }
__device__ __forceinline__ int perm32(int i) { return (i & 16) | perm16(i & 15); }
// Chunk-slot swizzles of the K rows and V rows: the 32 rows a fragment read touches (rows
// perm32(lane) of K, dims lane of V, one chunk each) land on distinct banks in every 8-lane
// (128-byte) and 16-lane (256-byte) read phase.
template <int D>
__device__ __forceinline__ int pf_fk(int r) {
  if constexpr (D >= 128)
    return perm16(r & 15);
  else
    return (r & 3) ^ ((r >> 2) & 1) ^ ((r >> 1) & 4);
}
__device__ __forceinline__ int pf_gv(int dim) { return ((dim >> 1) & 3) ^ ((dim >> 3) & 1); }

template <int D>
constexpr int prefill_stage_bytes() {
  return 32 * 2 * D + D * 64;  // K (32 keys x D dims) + V (D dims x 32 keys), bf16
}

template <int D, int HPW, int S>
__global__ __launch_bounds__(256) void prefill_attn_kernel(const bf16* __restrict__ qkv, const bf16* __restrict__ kpool,
                                                           const bf16* __restrict__ vpool,
                                                           const int32_t* __restrict__ block_table, int max_blocks,
                                                           const PrefillItem* __restrict__ items, int n_items,
                                                           float* __restrict__ part_o, float* __restrict__ part_ml,
                                                           bf16* __restrict__ out, int n_q, int n_kv, float scale_log2) {
  constexpr int KT = 32;                       // keys per step
  constexpr int RB = 2 * D;                    // bytes of one key row of the K stage
  constexpr int CPR = D / 8;                   // 16-byte chunks per key row
  constexpr int K_BYTES = KT * RB;
  constexpr int STAGE = prefill_stage_bytes<D>();
  constexpr int K_L = K_BYTES / 16 / 256;      // direct loads per thread per stage: K, V
  constexpr int V_L = (STAGE - K_BYTES) / 16 / 256;
  constexpr int NL = K_L + V_L;
  constexpr int NS = D / 16;                   // 16-dim steps of q.k
  constexpr int NT = D / 32;                   // 32-dim tiles of the output
  static_assert(K_L >= 1 && V_L >= 1 && K_L * 4096 == K_BYTES && S >= 2 && S <= 8, "stage layout");
  typedef __attribute__((address_space(3))) void lds_void;
  extern __shared__ __align__(16) unsigned char smem[];

  const int hgroups = n_q / HPW;
  const int item_idx = blockIdx.x / hgroups;
  if (item_idx >= n_items) return;
  const int h0 = (blockIdx.x % hgroups) * HPW;
  const PrefillItem it = items[item_idx];
  const int G = n_q / n_kv, g = h0 / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int head = h0 + wave % HPW;
  const int ql = (wave / HPW) * 32 + col;  // query of the tile (this lane's column)
  const int qi = it.q_begin + ql;          // query of the request
  const bool qvalid = qi < it.q_len;
  const int width = (n_q + 2 * n_kv) * D;

  // Q^T fragments (B operand): column = this lane's query, dims 16 s + 8 hf .. + 7
  bf16x8 qf[NS];
  {
    const bf16* qrow = qkv + (size_t)(it.token0 + min(qi, it.q_len - 1)) * width + (size_t)head * D + hf * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + s * 16);
  }
  // the item's block ids, one per lane (an item spans at most 64 blocks)
  const int n_keys = it.prefix + it.q_len;
  const int last_blk = (n_keys - 1) >> 4;
  const int blk0 = it.key_begin >> 4;
  const int my_blk = block_table[(size_t)it.req * max_blocks + min(blk0 + lane, last_blk)];
  const int nsteps = (it.key_end - it.key_begin + KT - 1) / KT;

  // this thread's share of a stage: K chunk (row, global chunk), V chunk (dim, key octet);
  // each lies in the step's first or second block (k_hi / v_hi)
  int k_off[K_L], v_off[V_L];
  bool k_hi[K_L], v_hi[V_L];
#pragma unroll
  for (int i = 0; i < K_L; ++i) {
    const int sl = (i * 4 + wave) * 64 + lane;
    const int r = sl / CPR, c = (sl % CPR) ^ pf_fk<D>(r);
    k_hi[i] = r >= kBlock;
    k_off[i] = (r & 15) * 32 + (c >> 2) * (kBlock * 32) + (c & 3) * 8;  // within [D/32][16 tokens][32 dims]
  }
#pragma unroll
  for (int i = 0; i < V_L; ++i) {
    const int sl = (i * 4 + wave) * 64 + lane;
    const int dim = sl >> 2, q = (sl & 3) ^ pf_gv(dim);
    v_hi[i] = (q >> 1) != 0;
    v_off[i] = dim * kBlock + (q & 1) * 8;  // within [D][16 tokens]
  }
  const bf16* kbase = kpool + (size_t)g * (kBlock * D);
  const bf16* vbase = vpool + (size_t)g * (D * kBlock);
  const size_t blk_stride = (size_t)n_kv * kBlock * D;
  auto issue = [&](int t) {
    unsigned char* base = smem + (t % S) * STAGE;
    // the step's two blocks (past the request's last block: its last one again, masked);
    // the lane index is wave-uniform, so the ids are scalar
    const int b0 = (it.key_begin >> 4) + 2 * t;
    const int ia = min(min(b0, last_blk), blk0 + 63) - blk0, ib = min(min(b0 + 1, last_blk), blk0 + 63) - blk0;
    const size_t pa = (size_t)__builtin_amdgcn_readlane(my_blk, ia) * blk_stride;
    const size_t pb = (size_t)__builtin_amdgcn_readlane(my_blk, ib) * blk_stride;
#pragma unroll
    for (int i = 0; i < K_L; ++i) {
      const bf16* src = kbase + (k_hi[i] ? pb : pa) + k_off[i];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)((unsigned char __attribute__((address_space(3)))*)(
                                                             (lds_void*)base) + (i * 4 + wave) * 64 * 16),
                                       16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V_L; ++i) {
      const bf16* src = vbase + (v_hi[i] ? pb : pa) + v_off[i];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)((unsigned char __attribute__((address_space(3)))*)(
                                                             (lds_void*)base) + K_BYTES + (i * 4 + wave) * 64 * 16),
                                       16, 0, 0);
    }
  };
  // wait until stage t has landed, with `newer` later stages of this thread still in flight
  auto wait_stage = [&](int newer) {
    switch (newer) {
      case 0: return wait_vmcnt<0>();
      case 1: return wait_vmcnt<NL * (S > 2 ? 1 : 0)>();
      case 2: return wait_vmcnt<NL * (S > 3 ? 2 : 0)>();
      case 3: return wait_vmcnt<NL * (S > 4 ? 3 : 0)>();
      case 4: return wait_vmcnt<NL * (S > 5 ? 4 : 0)>();
      case 5: return wait_vmcnt<NL * (S > 6 ? 5 : 0)>();
      default: return wait_vmcnt<NL * (S > 7 ? 6 : 0)>();
    }
  };

  // running reference m (log2 domain) and sum l per query; O^T accumulators. m is raised
  // only when a step's maximum exceeds it by more than kSlack (then O and l are rescaled):
  // the weights 2^(s - m) stay below 2^kSlack, and the result o / l does not depend on m
  constexpr float kSlack = 8.0f;
  float m = -INFINITY, l = 0.0f;
  f32x16 o[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[tt][r] = 0.0f;
  // keys below kend are visible to this lane's query: causal limit and the item's range;
  // steps ending at or below kfull (the wave's first query) need no mask
  const int kend = min(it.prefix + qi + 1, it.key_end);
  const int kfull = min(it.prefix + it.q_begin + (wave / HPW) * 32 + 1, it.key_end);
  const int prow = perm32(col);
  const int k_frag = prow * RB, k_swz = pf_fk<D>(prow);

  // one step: S^T = K Q^T, online softmax, O^T += V^T P^T. MASKED: some key of the step is
  // past the causal limit of a query of this wave or past the item's range; then keys past
  // the request's last one may also be in the stage (tail)
  auto step = [&](const unsigned char* kb, int key0, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const unsigned char* vb = kb + K_BYTES;
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + k_frag + (((2 * s + hf) ^ k_swz) * 16));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
    }
    // register r of lane half hf holds key key0 + 16 (r / 8) + 8 hf + r % 8
    if constexpr (MASKED) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + ((r & 8) << 1) + 8 * hf + (r & 7) >= kend) sacc[r] = -INFINITY;
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    if (__any(mx > m + kSlack)) {
      const float m_new = fmaxf(m, mx);
      const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= corr;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) o[tt] *= corr;
    }
    // a query whose keys are all masked so far keeps m = -inf: 0 as the reference then
    const float ref = m == -INFINITY ? 0.0f : m;
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], scale_log2, -ref));
      l += p;
      pf[r >> 3][r & 7] = (bf16)p;
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int dim = tt * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 vf = *reinterpret_cast<const bf16x8*>(vb + dim * 64 + (((2 * ks + hf) ^ pf_gv(dim)) * 16));
        if constexpr (MASKED) {
          // values of keys past the request's last one (unwritten slots of its last block)
          // are zeroed: their weight is 0, but 0 x NaN would poison O
          if (key0 + KT > n_keys) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (key0 + 16 * ks + 8 * hf + e >= n_keys) vf[e] = (bf16)0.0f;
          }
        }
        o[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[tt], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nsteps) issue(t);
  for (int t = 0; t < nsteps; ++t) {
    wait_stage(min(S - 2, nsteps - 1 - t));
    lds_barrier();  // stage t is in LDS for every wave; every wave is done with stage t - 1
    if (t + S - 1 < nsteps) issue(t + S - 1);
    const unsigned char* kb = smem + (t % S) * STAGE;
    const int key0 = it.key_begin + t * KT;
    if (key0 + KT <= kfull)
      step(kb, key0, std::false_type{});
    else
      step(kb, key0, std::true_type{});
  }

  l += __shfl_xor(l, 32, 64);
  if (!qvalid) return;
  // lane half hf holds dims 32 tt + 8 j + 4 hf .. + 3 in registers 4 j .. 4 j + 3
  if (it.part < 0) {
    const float inv = 1.0f / l;
    bf16* orow = out + (size_t)(it.token0 + qi) * n_q * D + (size_t)head * D + 4 * hf;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[tt][4 * j + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + tt * 32 + 8 * j) = v;
      }
  } else {
    const size_t slot = (size_t)(it.part + ql * it.n_chunks) * n_q + head;
    float* po = part_o + slot * D + 4 * hf;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(po + tt * 32 + 8 * j) =
            f32x4{o[tt][4 * j], o[tt][4 * j + 1], o[tt][4 * j + 2], o[tt][4 * j + 3]};
    if (hf == 0) {
      part_ml[slot * 2 + 0] = m;
      part_ml[slot * 2 + 1] = l;
    }
  }
}

template <int D, int HPW>
static void launch_prefill_t(int grid, hipStream_t s, const bf16* qkv, const bf16* kpool, const bf16* vpool,
                             const int32_t* block_table, int max_blocks, const PrefillItem* items, int n_items,
                             float* part_o, float* part_ml, bf16* out, int n_q, int n_kv, float scale_log2) {
  constexpr int S = NF_PF_STAGES;  // LDS stages of 32 keys (16 KB each at head_dim 128)
  if constexpr (S * prefill_stage_bytes<D>() > 65536) {
    static bool attr_set = false;
    if (!attr_set) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_attn_kernel<D, HPW, S>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, S * prefill_stage_bytes<D>());
      attr_set = true;
    }
  }
  hipLaunchKernelGGL((prefill_attn_kernel<D, HPW, S>), dim3(grid), dim3(256), S * prefill_stage_bytes<D>(), s, qkv,
                     kpool, vpool, block_table, max_blocks, items, n_items, part_o, part_ml, out, n_q, n_kv,
                     scale_log2);
}

hipError_t launch_prefill_attn(const bf16* qkv, const bf16* kpool, const bf16* vpool, const int32_t* block_table,
                               int max_blocks, const PrefillItem* items, int n_items, const CombineItem* combines,
                               int n_combines, float* part_o, float* part_ml, bf16* out, int n_q, int n_kv, int d,
                               hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  const int hpw = prefill_heads_per_wg(n_q / n_kv);
  const int grid = n_items * (n_q / hpw);
#define NF_PREFILL_CASE(D_, H_)                                                                                \
  if (d == D_ && hpw == H_)                                                                                    \
    launch_prefill_t<D_, H_>(grid, s, qkv, kpool, vpool, block_table, max_blocks, items, n_items, part_o,     \
                             part_ml, out, n_q, n_kv, scale_log2);                                             \
  else
  NF_PREFILL_CASE(128, 4)
  NF_PREFILL_CASE(128, 2)
  NF_PREFILL_CASE(128, 1)
  NF_PREFILL_CASE(64, 4)
  NF_PREFILL_CASE(64, 2)
  NF_PREFILL_CASE(64, 1)
  return hipErrorInvalidValue;
#undef NF_PREFILL_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_combines <= 0) return e;
  return launch_decode_combine(combines, n_combines, part_o, part_ml, out, n_q, n_kv, d, s);
}

}  // namespace nf
