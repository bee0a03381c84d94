// Paged GQA decode attention on gfx950 matrix cores (memory-bound, one query per request;
// NanoFlow summary page, memory-bound operations: decode attention streams the per-request
// KV-cache). Prefill attention is in nf_prefill.hip.
//
// One wave owns 16 "columns" — the query heads sharing one KV head, one query per request —
// and streams 16-token KV blocks through the block table. Per block: S^T[16 keys][16 cols] = K_blk Q^T with 16x16x32 bf16 MFMAs over head_dim,
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

// The request's newest key (sequence position pos) taken from its row of qkv instead of the
// pool: a virtual block whose key row 0 holds the rotated k and whose value column 0 holds v,
// every other key masked (and its value zero).
template <int D>
__device__ __forceinline__ void attend_new_key(AttnState<D>& st, const bf16x8* qf, const bf16* __restrict__ krow,
                                               const bf16* __restrict__ vrow, int pos, float scale_log2, int lane) {
  const int i16 = lane & 15, grp = lane >> 4;
  KvFrag<D> f[1];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    if (i16 == 0) {
      f[0].k[c] = *reinterpret_cast<const bf16x8*>(krow + c * 32 + grp * 8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[0].k[c][j] = (bf16)0.0f;
    }
  }
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
#pragma unroll
    for (int r = 0; r < 4; ++r) f[0].v[dc][r] = (bf16)0.0f;
    if (grp == 0) f[0].v[dc][0] = vrow[dc * 16 + i16];
  }
  attend_group<D, 1>(st, f, qf, pos, pos, scale_log2, grp);
}

// ---------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------

// Waves take work units (item, KV head) in strides of the grid's wave count, so a grid
// smaller than the work keeps a bounded footprint (the memory nano-op's resource share)
// while each wave streams many blocks. With new_from_qkv the newest key of each request
// (position n_keys - 1) is read from the request's qkv row (rotated k, v), not from the
// pool: the layer appends the decode tokens' K/V to the pool after this kernel, since a
// launch that reads pool lines just partially written by the append runs 3-6% slower.
template <int D, int NB, int R>
__global__ __launch_bounds__(256) void decode_attn_kernel(const bf16* __restrict__ qkv, const bf16* __restrict__ kpool,
                                                          const bf16* __restrict__ vpool,
                                                          const int32_t* __restrict__ block_table, int max_blocks,
                                                          const DecodeItem* __restrict__ items, int n_items,
                                                          float* __restrict__ part_o, float* __restrict__ part_ml,
                                                          bf16* __restrict__ out, int n_q, int n_kv, float scale_log2,
                                                          int new_from_qkv) {
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
    if (new_from_qkv) {
      const int n_pool = it.n_keys - 1;  // keys already in the pool
      const int b1 = min(it.blk_end, (n_pool + kBlock - 1) / kBlock);
      attend_range<D, NB, R>(st, qf, block_table + (size_t)it.req * max_blocks, it.blk_begin, b1, kpool, vpool, n_kv,
                            g, n_pool - 1, n_pool, scale_log2, lane);
      if (it.blk_end * kBlock >= it.n_keys) {  // this item holds the request's last block
        const bf16* row = qkv + (size_t)it.token * width;
        attend_new_key<D>(st, qf, row + (size_t)(n_q + g) * D, row + (size_t)(n_q + n_kv + g) * D, n_pool, scale_log2,
                          lane);
      }
    } else {
      attend_range<D, NB, R>(st, qf, block_table + (size_t)it.req * max_blocks, it.blk_begin, it.blk_end, kpool,
                            vpool, n_kv, g, it.n_keys - 1, it.n_keys, scale_log2, lane);
    }
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

// ev_start / ev_stop (both or neither): timing events recorded by the dispatch itself
// (no marker packets between this kernel and its neighbours on the stream).
template <int D, int NB, int R>
static void launch_decode_t(int grid, hipStream_t s, const bf16* qkv, const bf16* kpool, const bf16* vpool,
                            const int32_t* block_table, int max_blocks, const DecodeItem* items, int n_items,
                            float* part_o, float* part_ml, bf16* out, int n_q, int n_kv, float scale_log2,
                            int new_from_qkv, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (ev_start)
    hipExtLaunchKernelGGL((decode_attn_kernel<D, NB, R>), dim3(grid), dim3(256), 0, s, ev_start, ev_stop, 0, qkv,
                          kpool, vpool, block_table, max_blocks, items, n_items, part_o, part_ml, out, n_q, n_kv,
                          scale_log2, new_from_qkv);
  else
    hipLaunchKernelGGL((decode_attn_kernel<D, NB, R>), dim3(grid), dim3(256), 0, s, qkv, kpool, vpool, block_table,
                       max_blocks, items, n_items, part_o, part_ml, out, n_q, n_kv, scale_log2, new_from_qkv);
}

// Supported (blocks per softmax step, ring depth) pairs.
template <int D>
static hipError_t launch_decode_d(int nb, int ring, int grid, hipStream_t s, const bf16* qkv, const bf16* kpool,
                                  const bf16* vpool, const int32_t* block_table, int max_blocks,
                                  const DecodeItem* items, int n_items, float* part_o, float* part_ml, bf16* out,
                                  int n_q, int n_kv, float scale_log2, int new_from_qkv, hipEvent_t ev_start,
                                  hipEvent_t ev_stop) {
#define NF_DECODE_CASE(NB_, R_)                                                                                 \
  if (nb == NB_ && ring == R_) {                                                                                \
    launch_decode_t<D, NB_, R_>(grid, s, qkv, kpool, vpool, block_table, max_blocks, items, n_items, part_o,    \
                                part_ml, out, n_q, n_kv, scale_log2, new_from_qkv, ev_start, ev_stop);          \
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
  return (nb == 0 && ring == 0) || (nb == 1 && ring >= 2 && ring <= 4) || (nb == 2 && (ring == 2 || ring == 3));
}

// The automatic launch shape (nb = 0): the default kernel (1 block per step, ring of 2) holds
// 3 waves per SIMD. Work of fewer waves than one round of those slots (a KV head per GPU
// with long contexts: a few thousand units) leaves most slots empty, so each wave then
// streams 2 blocks per step instead (2 waves per SIMD, twice the bytes in flight per wave);
// measured in the 70B tensor-parallel share's layer: 316 -> 303 us, while the 8B layer's
// 12.8k units keep the default (1229 against 1240 us).
static void decode_auto_config(int waves, int& nb, int& ring) {
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  nb = waves < n_cu * 4 * 3 ? 2 : 1;
  ring = 2;
}

// nb: KV blocks per softmax step (0 = chosen from the work, with ring 0); ring: register
// buffers of nb blocks (ring - 1 groups in flight); max_grid: workgroup cap (0 = one wave
// per unit)
hipError_t launch_decode_attn(const bf16* qkv, const bf16* kpool, const bf16* vpool, const int32_t* block_table,
                              int max_blocks, const DecodeItem* items, int n_items, float* part_o, float* part_ml,
                              bf16* out, int n_q, int n_kv, int d, int max_grid, int nb, int ring, hipStream_t s,
                              hipEvent_t ev_start, hipEvent_t ev_stop, int new_from_qkv) {
  if (n_items <= 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  const int waves = n_items * n_kv;
  if (nb == 0) decode_auto_config(waves, nb, ring);
  int grid = (waves + 3) / 4;
  if (max_grid > 0 && grid > max_grid) grid = max_grid;
  if (d == 128)
    return launch_decode_d<128>(nb, ring, grid, s, qkv, kpool, vpool, block_table, max_blocks, items, n_items, part_o,
                                part_ml, out, n_q, n_kv, scale_log2, new_from_qkv, ev_start, ev_stop);
  if (d == 64)
    return launch_decode_d<64>(nb, ring, grid, s, qkv, kpool, vpool, block_table, max_blocks, items, n_items, part_o,
                               part_ml, out, n_q, n_kv, scale_log2, new_from_qkv, ev_start, ev_stop);
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

}  // namespace nf
