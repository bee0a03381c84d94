// Paged causal GQA attention on gfx950 matrix cores: decode attention (memory-bound, one
// query per request; NanoFlow summary page, memory-bound operations: decode attention
// streams the per-request KV-cache) and prefill attention (compute-bound, causal within a
// request; "Inside nano-vLLM", prefill batching keeps request boundaries).
//
// One wave owns 16 "columns" and streams 16-token KV blocks through the block table:
//   decode : columns = the query heads sharing one KV head, one query per request
//   prefill: columns = 16 consecutive queries of one query head
// Per block: S^T[16 keys][16 cols] = K_blk Q^T with 16x16x32 bf16 MFMAs over head_dim,
// an online softmax per column (base-2 exponent, running max and sum), then
// O^T[d][16 cols] += V_blk^T P^T with 16x16x16 bf16 MFMAs. K is stored in 32-dim column
// chunks, each token-major, so a lane's 8 consecutive dims are one 16-byte load and one
// wave instruction reads 16 tokens x 64 bytes = 1 KB of whole lines; V is dim-major within
// a block, so a lane's 4 consecutive keys of one dim are one 8-byte load — both already in
// the operand layout of the matrix instruction, no LDS transpose needed.
//
// Decode work is split along the KV sequence (split-KV): each wave takes a bounded run of
// blocks of one request and one KV head; multi-chunk requests write unnormalised partial
// outputs plus (max, sum) and a combine kernel merges them.
#include "nf_internal.h"

namespace nf {

__device__ __forceinline__ float wave_max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// State of one wave's 16 columns: running max m (log2 domain), partial sum l of this lane's
// keys, and O^T accumulators (lane holds dims dc*16 + 4*grp + r of column lane%16).
template <int D>
struct AttnState {
  float m;
  float l;
  f32x4 o[D / 16];
};

template <int D>
struct KvFrag {
  bf16x8 k[D / 32];
  bf16x4 v[D / 16];
};

// K/V are streamed once per iteration: nontemporal loads keep them from displacing the
// GEMMs' weight tiles in L2 and the last-level cache while both run.
template <int D>
__device__ __forceinline__ void load_block(KvFrag<D>& f, const bf16* __restrict__ kpool, const bf16* __restrict__ vpool,
                                           int blk, int n_kv, int g, int i16, int grp) {
  const bf16* kb = kpool + ((size_t)blk * n_kv + g) * (kBlock * D);
  const bf16* vb = vpool + ((size_t)blk * n_kv + g) * (D * kBlock);
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    f.k[c] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(kb + c * (kBlock * 32) + i16 * 32 + grp * 8));
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    f.v[dc] = __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(vb + (dc * 16 + i16) * kBlock + grp * 4));
}

// Process NB consecutive blocks (16*NB keys starting at sequence position key0) in one
// online-softmax step: the NB score tiles are independent MFMAs, then one running-max /
// rescale update for all of them, then the NB value products. Column limit: key k is
// visible to this lane's column iff k <= limit.
template <int D, int NB>
__device__ __forceinline__ void attend_group(AttnState<D>& st, const KvFrag<D> (&f)[NB], const bf16x8* qf, int key0,
                                             int limit, float scale_log2, int grp) {
  float sv[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[j].k[c], qf[c], s, 0, 0, 0);
    const int kbase = key0 + j * kBlock + grp * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[j][r] = (kbase + r <= limit) ? s[r] * scale_log2 : -INFINITY;
  }
  float bm = -INFINITY;
#pragma unroll
  for (int j = 0; j < NB; ++j) bm = fmaxf(bm, fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3])));
  bm = wave_max16(bm);
  const float m_new = fmaxf(st.m, bm);
  // a column whose keys are all masked so far keeps m = -inf; use 0 as the reference then
  const float ref = (m_new == -INFINITY) ? 0.0f : m_new;
  const float corr = exp2f(st.m - ref);
  st.m = m_new;
  bf16x4 pf[NB];
  float lsum = 0.0f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = exp2f(sv[j][r] - ref);
      lsum += p;
      pf[j][r] = (bf16)p;
    }
  st.l = st.l * corr + lsum;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) st.o[dc] *= corr;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      st.o[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(f[j].v[dc], pf[j], st.o[dc], 0, 0, 0);
}

template <int D, int NB>
__device__ __forceinline__ void load_group(KvFrag<D> (&f)[NB], const bf16* __restrict__ kpool,
                                           const bf16* __restrict__ vpool, int my_blk, int b, int nb, int n_kv, int g,
                                           int i16, int grp) {
#pragma unroll
  for (int j = 0; j < NB; ++j) load_block<D>(f[j], kpool, vpool, __shfl(my_blk, min(b + j, nb - 1), 64), n_kv, g, i16, grp);
}

// Keeps the compiler from moving the loads issued before it past the math after it, and
// the math of a later group above it (the scheduler would otherwise pull the next group's
// MFMAs forward, which waits for the loads just issued and empties the pipe every trip).
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Walk logical blocks [b0, b1) of block-table row `bt_row` (a request with n_keys keys).
// Full blocks stream in groups of NB through a ring of R register buffers: while one group
// is multiplied, the next R-1 groups are in flight. The loop body has no branches, which
// keeps the compiler's memory wait counts exact: loads past the range repeat its last block
// (a cache hit) and those phantom blocks are masked out. A partial last block is handled
// after the loop, with the values of keys past the sequence end zeroed so that stale pool
// contents cannot leak through 0 * NaN.
template <int D, int NB, int R>
__device__ __forceinline__ void attend_range(AttnState<D>& st, const bf16x8* qf, const int32_t* __restrict__ bt_row,
                                             int b0, int b1, const bf16* __restrict__ kpool,
                                             const bf16* __restrict__ vpool, int n_kv, int g, int limit, int n_keys,
                                             float scale_log2, int lane) {
  static_assert(R >= 2, "ring of at least two buffers");
  const int i16 = lane & 15, grp = lane >> 4;
  const int e = min(b1, n_keys / kBlock);  // full blocks: [b0, e)
  for (int base = b0; base < e; base += 64) {
    const int nb = min(64, e - base);
    const int my_blk = bt_row[base + min(lane, nb - 1)];
    // phantom blocks past this batch of (at most 64) blocks are masked out here, also when
    // the range continues in the next batch
    const int ring_limit = min(limit, (base + nb) * kBlock - 1);
    KvFrag<D> f[R][NB];
#pragma unroll
    for (int i = 0; i < R - 1; ++i) load_group<D, NB>(f[i], kpool, vpool, my_blk, i * NB, nb, n_kv, g, i16, grp);
    for (int b = 0; b < nb; b += R * NB) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        load_group<D, NB>(f[(i + R - 1) % R], kpool, vpool, my_blk, b + (i + R - 1) * NB, nb, n_kv, g, i16, grp);
        issue_fence();
        attend_group<D, NB>(st, f[i], qf, (base + b + i * NB) * kBlock, ring_limit, scale_log2, grp);
      }
    }
  }
  if (b1 > e) {
    KvFrag<D> f[1];
    load_block<D>(f[0], kpool, vpool, bt_row[e], n_kv, g, i16, grp);
    const int kbase = e * kBlock + grp * 4;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kbase + r >= n_keys) f[0].v[dc][r] = (bf16)0.0f;
    attend_group<D, 1>(st, f, qf, e * kBlock, limit, scale_log2, grp);
  }
}

template <int D>
__device__ __forceinline__ void init_state(AttnState<D>& st) {
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) st.o[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------

// Waves take work units (item, KV head) in strides of the grid's wave count, so a grid
// smaller than the work keeps a bounded footprint (the memory nano-op's resource share)
// while each wave streams many blocks.
template <int D, int NB, int R>
__global__ __launch_bounds__(256) void decode_attn_kernel(const bf16* __restrict__ qkv, const bf16* __restrict__ kpool,
                                                          const bf16* __restrict__ vpool,
                                                          const int32_t* __restrict__ block_table, int max_blocks,
                                                          const DecodeItem* __restrict__ items, int n_items,
                                                          float* __restrict__ part_o, float* __restrict__ part_ml,
                                                          bf16* __restrict__ out, int n_q, int n_kv, float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int n_waves = gridDim.x * 4;
  const int G = n_q / n_kv;
  const int i16 = lane & 15, grp = lane >> 4;
  const int width = (n_q + 2 * n_kv) * D;
  for (int wg = blockIdx.x * 4 + (threadIdx.x >> 6); wg < n_items * n_kv; wg += n_waves) {
    const int item_idx = wg / n_kv;
    const int g = wg % n_kv;
    const DecodeItem it = items[item_idx];
    bf16x8 qf[D / 32];
    {
      const bf16* qrow = qkv + (size_t)it.token * width + (size_t)(g * G + i16) * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        if (i16 < G) {
          qf[c] = *reinterpret_cast<const bf16x8*>(qrow + c * 32 + grp * 8);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) qf[c][j] = (bf16)0.0f;
        }
      }
    }
    AttnState<D> st;
    init_state<D>(st);
    attend_range<D, NB, R>(st, qf, block_table + (size_t)it.req * max_blocks, it.blk_begin, it.blk_end, kpool, vpool,
                          n_kv, g, it.n_keys - 1, it.n_keys, scale_log2, lane);
    const float l = wave_sum16(st.l);
    if (i16 < G) {
      if (it.part < 0) {
        const float inv = 1.0f / l;
        bf16* orow = out + (size_t)it.token * n_q * D + (size_t)(g * G + i16) * D;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          bf16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (bf16)(st.o[dc][r] * inv);
          *reinterpret_cast<bf16x4*>(orow + dc * 16 + grp * 4) = o;
        }
      } else {
        const size_t pbase = ((size_t)it.part * n_kv + g) * G + i16;
        float* po = part_o + pbase * D;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) *reinterpret_cast<f32x4*>(po + dc * 16 + grp * 4) = st.o[dc];
        if (grp == 0) {
          part_ml[pbase * 2 + 0] = st.m;
          part_ml[pbase * 2 + 1] = l;
        }
      }
    }
  }
}

// Merge split-KV partials: o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// One wave per (request, query head): lane p holds part p's (m, l) (64 parts per round),
// then the weighted sum over parts streams each part's D-vector as one coalesced row.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const CombineItem* __restrict__ items, int n_items,
                                                             const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml, bf16* __restrict__ out,
                                                             int n_q, int n_kv) {
  constexpr int PER = D / 64;  // outputs per lane
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int item_idx = wid / n_q;
  const int hq = wid % n_q;  // query head
  if (item_idx >= n_items) return;
  const CombineItem it = items[item_idx];
  const int G = n_q / n_kv;
  const int g = hq / G, h = hq % G;
  auto slot = [&](int p) { return ((size_t)(it.part_begin + p) * n_kv + g) * G + h; };
  float M = -INFINITY;
  for (int p0 = 0; p0 < it.n_parts; p0 += 64)
    if (p0 + lane < it.n_parts) M = fmaxf(M, part_ml[slot(p0 + lane) * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float L = 0.0f, acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
  for (int p0 = 0; p0 < it.n_parts; p0 += 64) {
    const int np = min(64, it.n_parts - p0);
    float wgt = 0.0f;
    if (lane < np) {
      const size_t sl = slot(p0 + lane);
      wgt = exp2f(part_ml[sl * 2] - M);
      L += wgt * part_ml[sl * 2 + 1];
    }
#pragma unroll 4
    for (int q = 0; q < np; ++q) {
      const float w = __shfl(wgt, q, 64);
      const float* po = part_o + slot(p0 + q) * D + lane * PER;
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += w * po[j];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
  const float inv = 1.0f / L;
  bf16* orow = out + (size_t)it.token * n_q * D + (size_t)hq * D + lane * PER;
#pragma unroll
  for (int j = 0; j < PER; ++j) orow[j] = (bf16)(acc[j] * inv);
}

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
  static_assert(K_L >= 1 && V_L >= 1 && K_L * 4096 == K_BYTES && S >= 2 && S <= 4, "stage layout");
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

  // this thread's share of a stage: K chunk (row, global chunk), V chunk (dim, key octet)
  int k_row[K_L], k_off[K_L], v_q[V_L], v_off[V_L];
#pragma unroll
  for (int i = 0; i < K_L; ++i) {
    const int sl = (i * 4 + wave) * 64 + lane;
    const int r = sl / CPR, c = (sl % CPR) ^ pf_fk<D>(r);
    k_row[i] = r;
    k_off[i] = (c >> 2) * (kBlock * 32) + (c & 3) * 8;  // within [D/32][16 tokens][32 dims]
  }
#pragma unroll
  for (int i = 0; i < V_L; ++i) {
    const int sl = (i * 4 + wave) * 64 + lane;
    const int dim = sl >> 2, q = (sl & 3) ^ pf_gv(dim);
    v_q[i] = q;
    v_off[i] = dim * kBlock + (q & 1) * 8;  // within [D][16 tokens]
  }
  auto issue = [&](int t) {
    unsigned char* base = smem + (t % S) * STAGE;
    const int key0 = it.key_begin + t * KT;
#pragma unroll
    for (int i = 0; i < K_L; ++i) {
      const int key = key0 + k_row[i];
      const int lb = min(min(key >> 4, last_blk), blk0 + 63);
      const int phys = __shfl(my_blk, lb - blk0, 64);
      const bf16* src = kpool + ((size_t)phys * n_kv + g) * (kBlock * D) + (key & 15) * 32 + k_off[i];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)((unsigned char __attribute__((address_space(3)))*)(
                                                             (lds_void*)base) + (i * 4 + wave) * 64 * 16),
                                       16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V_L; ++i) {
      const int lb = min(min((key0 >> 4) + (v_q[i] >> 1), last_blk), blk0 + 63);
      const int phys = __shfl(my_blk, lb - blk0, 64);
      const bf16* src = vpool + ((size_t)phys * n_kv + g) * (D * kBlock) + v_off[i];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)((unsigned char __attribute__((address_space(3)))*)(
                                                             (lds_void*)base) + K_BYTES + (i * 4 + wave) * 64 * 16),
                                       16, 0, 0);
    }
  };
  // wait until stage t has landed, with `newer` later stages of this thread still in flight
  auto wait_stage = [&](int newer) {
    if constexpr (S > 3) {
      if (newer >= 2) return wait_vmcnt<NL * 2>();
    }
    if constexpr (S > 2) {
      if (newer >= 1) return wait_vmcnt<NL>();
    }
    wait_vmcnt<0>();
  };

  float m = -INFINITY, l = 0.0f;
  f32x16 o[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[tt][r] = 0.0f;
  // keys below kend are visible to this lane's query: causal limit and the item's range
  const int kend = min(it.prefix + qi + 1, it.key_end);
  const int prow = perm32(col);
  const int k_frag = prow * RB, k_swz = pf_fk<D>(prow);

#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nsteps) issue(t);
  for (int t = 0; t < nsteps; ++t) {
    wait_stage(min(S - 2, nsteps - 1 - t));
    lds_barrier();  // stage t is in LDS for every wave; every wave is done with stage t - 1
    if (t + S - 1 < nsteps) issue(t + S - 1);
    const unsigned char* kb = smem + (t % S) * STAGE;
    const unsigned char* vb = kb + K_BYTES;
    const int key0 = it.key_begin + t * KT;

    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + k_frag + (((2 * s + hf) ^ k_swz) * 16));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
    }
    // online softmax in base 2; register r of lane half hf holds key 16 (r / 8) + 8 hf + r % 8
    float sv[16], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + ((r & 8) << 1) + 8 * hf + (r & 7);
      sv[r] = key < kend ? sacc[r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    // a query whose keys are all masked so far keeps m = -inf; use 0 as the reference then
    const float ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float corr = __builtin_amdgcn_exp2f(m - ref);
    m = m_new;
    bf16x8 pf[2];
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(sv[r] - ref);
      ls += p;
      pf[r >> 3][r & 7] = (bf16)p;
    }
    l = l * corr + ls;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) o[tt] *= corr;
    // values of keys past the request's last one (unwritten slots of its last block) are
    // zeroed: their weight is 0, but 0 x NaN would poison O
    const bool tail = key0 + KT > n_keys;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int dim = tt * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 vf = *reinterpret_cast<const bf16x8*>(vb + dim * 64 + (((2 * ks + hf) ^ pf_gv(dim)) * 16));
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (key0 + 16 * ks + 8 * hf + e >= n_keys) vf[e] = (bf16)0.0f;
        }
        o[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[tt], 0, 0, 0);
      }
    }
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

// ---------------------------------------------------------------------------------------

template <int D, int NB, int R>
static void launch_decode_t(int grid, hipStream_t s, const bf16* qkv, const bf16* kpool, const bf16* vpool,
                            const int32_t* block_table, int max_blocks, const DecodeItem* items, int n_items,
                            float* part_o, float* part_ml, bf16* out, int n_q, int n_kv, float scale_log2) {
  hipLaunchKernelGGL((decode_attn_kernel<D, NB, R>), dim3(grid), dim3(256), 0, s, qkv, kpool, vpool, block_table,
                     max_blocks, items, n_items, part_o, part_ml, out, n_q, n_kv, scale_log2);
}

// Supported (blocks per softmax step, ring depth) pairs.
template <int D>
static hipError_t launch_decode_d(int nb, int ring, int grid, hipStream_t s, const bf16* qkv, const bf16* kpool,
                                  const bf16* vpool, const int32_t* block_table, int max_blocks,
                                  const DecodeItem* items, int n_items, float* part_o, float* part_ml, bf16* out,
                                  int n_q, int n_kv, float scale_log2) {
#define NF_DECODE_CASE(NB_, R_)                                                                                 \
  if (nb == NB_ && ring == R_) {                                                                                \
    launch_decode_t<D, NB_, R_>(grid, s, qkv, kpool, vpool, block_table, max_blocks, items, n_items, part_o,    \
                                part_ml, out, n_q, n_kv, scale_log2);                                           \
    return hipGetLastError();                                                                                   \
  }
  NF_DECODE_CASE(1, 2)
  NF_DECODE_CASE(1, 3)
  NF_DECODE_CASE(1, 4)
  NF_DECODE_CASE(2, 2)
  NF_DECODE_CASE(2, 3)
#undef NF_DECODE_CASE
  return hipErrorInvalidValue;
}

bool decode_config_supported(int nb, int ring) {
  return (nb == 1 && ring >= 2 && ring <= 4) || (nb == 2 && (ring == 2 || ring == 3));
}

// nb: KV blocks per softmax step; ring: register buffers of nb blocks (ring - 1 groups in
// flight); max_grid: workgroup cap (0 = one wave per unit)
hipError_t launch_decode_attn(const bf16* qkv, const bf16* kpool, const bf16* vpool, const int32_t* block_table,
                              int max_blocks, const DecodeItem* items, int n_items, float* part_o, float* part_ml,
                              bf16* out, int n_q, int n_kv, int d, int max_grid, int nb, int ring, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  const int waves = n_items * n_kv;
  int grid = (waves + 3) / 4;
  if (max_grid > 0 && grid > max_grid) grid = max_grid;
  if (d == 128)
    return launch_decode_d<128>(nb, ring, grid, s, qkv, kpool, vpool, block_table, max_blocks, items, n_items, part_o,
                                part_ml, out, n_q, n_kv, scale_log2);
  if (d == 64)
    return launch_decode_d<64>(nb, ring, grid, s, qkv, kpool, vpool, block_table, max_blocks, items, n_items, part_o,
                               part_ml, out, n_q, n_kv, scale_log2);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const CombineItem* combines, int n_combines, const float* part_o,
                                 const float* part_ml, bf16* out, int n_q, int n_kv, int d, hipStream_t s) {
  if (n_combines <= 0) return hipSuccess;
  const int cgrid = (n_combines * n_q + 3) / 4;
  if (d == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(cgrid), dim3(256), 0, s, combines, n_combines, part_o,
                       part_ml, out, n_q, n_kv);
  else if (d == 64)
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(cgrid), dim3(256), 0, s, combines, n_combines, part_o,
                       part_ml, out, n_q, n_kv);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D, int HPW>
static void launch_prefill_t(int grid, hipStream_t s, const bf16* qkv, const bf16* kpool, const bf16* vpool,
                             const int32_t* block_table, int max_blocks, const PrefillItem* items, int n_items,
                             float* part_o, float* part_ml, bf16* out, int n_q, int n_kv, float scale_log2) {
  constexpr int S = 3;  // LDS stages of 32 keys (48 KB at head_dim 128)
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
