// Row-wise memory-bound ops of the layer: RMSNorm, and rotary embedding fused with the
// paged KV append.
//
// RMSNorm (pre-attention and pre-FFN norm): out = x / sqrt(mean(x^2) + eps) * g.
// Rotary: rotate-half pairs (i, i + d/2) of every q and k head by angle pos * inv_freq[i];
// the rotated k and the value v of each token are stored at the token's paged-KV slot
// ("Inside nano-vLLM", paged KV: the slot mapping locates new KV stores; "LLM Inference
// Performance", PagedAttention block tables). Within a block, K is stored in 32-dim column
// chunks, each token-major, and V dim-major (the layouts the attention kernels read with
// matrix cores).
#include "nf_internal.h"

namespace nf {

// One workgroup of 256 threads per row; each thread owns CPT chunks of 8 contiguous
// elements (n <= 2048 CPT), loaded once and kept in registers for the scaling pass (0: any n,
// the row read twice).
template <int CPT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const bf16* __restrict__ x, const bf16* __restrict__ g,
                                                      bf16* __restrict__ out, int n, float eps) {
  const int row = blockIdx.x;
  const bf16* xr = x + (size_t)row * n;
  bf16* orow = out + (size_t)row * n;
  const int chunks = n / 8;
  constexpr int R = CPT > 0 ? CPT : 1;
  bf16x8 keep[R];
  float ss = 0.0f;
  if constexpr (CPT > 0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * 256;
      if (c < chunks) {
        keep[i] = *reinterpret_cast<const bf16x8*>(xr + c * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += (float)keep[i][j] * (float)keep[i][j];
      }
    }
  } else {
    for (int c = threadIdx.x; c < chunks; c += 256) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += (float)v[j] * (float)v[j];
    }
  }
  // wave reduction then across the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(total / (float)n + eps);
  auto scale = [&](int c, const bf16x8& v) {
    const bf16x8 gv = *reinterpret_cast<const bf16x8*>(g + c * 8);
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (bf16)(((float)v[j] * inv) * (float)gv[j]);
    *reinterpret_cast<bf16x8*>(orow + c * 8) = o;
  };
  if constexpr (CPT > 0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * 256;
      if (c < chunks) scale(c, keep[i]);
    }
  } else {
    for (int c = threadIdx.x; c < chunks; c += 256) scale(c, *reinterpret_cast<const bf16x8*>(xr + c * 8));
  }
}

hipError_t launch_rmsnorm(const bf16* x, const bf16* g, bf16* out, int m, int n, float eps, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  const int cpt = (n / 8 + 255) / 256;
  if (cpt <= 1)
    hipLaunchKernelGGL(rmsnorm_kernel<1>, dim3(m), dim3(256), 0, s, x, g, out, n, eps);
  else if (cpt == 2)
    hipLaunchKernelGGL(rmsnorm_kernel<2>, dim3(m), dim3(256), 0, s, x, g, out, n, eps);
  else if (cpt <= 4)
    hipLaunchKernelGGL(rmsnorm_kernel<4>, dim3(m), dim3(256), 0, s, x, g, out, n, eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<0>, dim3(m), dim3(256), 0, s, x, g, out, n, eps);
  return hipGetLastError();
}

// One workgroup per token. The token's angles pos * inv_freq[i] are evaluated once (d/2
// sincos, shared through LDS by its n_q + n_kv heads); then each thread rotates 8
// consecutive pairs (i0..i0+7, i0+d/2..i0+d/2+7) of one head with two 16-byte loads and two
// 16-byte stores: q and k in place in qkv, k also into the token's slot of the pool (8
// consecutive dims lie in one 32-dim column chunk). v is stored dim-major, one 2-byte
// element per dimension row of the block. Tokens below t_defer keep their K/V out of the
// pool here (kv_append_kernel stores them later, from qkv).
__global__ __launch_bounds__(256) void rope_kv_kernel(bf16* __restrict__ qkv, const int32_t* __restrict__ tok_pos,
                                                      const int32_t* __restrict__ tok_slot,
                                                      const float* __restrict__ inv_freq, bf16* __restrict__ kpool,
                                                      bf16* __restrict__ vpool, int t_begin, int t_defer, int n_q,
                                                      int n_kv, int d) {
  __shared__ float cs_l[128], sn_l[128];  // d / 2 <= 128
  const int t = t_begin + blockIdx.x;
  const bool append = t >= t_defer;
  const int pos = tok_pos[t];
  const int slot = tok_slot[t];
  const int blk = slot / kBlock, off = slot % kBlock;
  const int half = d / 2;
  const int width = (n_q + 2 * n_kv) * d;
  bf16* row = qkv + (size_t)t * width;
  for (int i = threadIdx.x; i < half; i += 256) {
    float sn, cs;
    sincosf((float)pos * inv_freq[i], &sn, &cs);  // full-range reduction (angles reach ~4096 rad)
    cs_l[i] = cs;
    sn_l[i] = sn;
  }
  __syncthreads();
  const int per_head = half / 8;
  const int n_chunks = (n_q + n_kv) * per_head;
  for (int c = threadIdx.x; c < n_chunks; c += 256) {
    const int head = c / per_head, i0 = (c % per_head) * 8;
    bf16* hp = row + head * d;
    const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(hp + i0);
    const bf16x8 x2 = *reinterpret_cast<const bf16x8*>(hp + i0 + half);
    bf16x8 o1, o2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float cs = cs_l[i0 + e], sn = sn_l[i0 + e];
      const float a = (float)x1[e], b = (float)x2[e];
      o1[e] = (bf16)(a * cs - b * sn);
      o2[e] = (bf16)(b * cs + a * sn);
    }
    *reinterpret_cast<bf16x8*>(hp + i0) = o1;
    *reinterpret_cast<bf16x8*>(hp + i0 + half) = o2;
    if (head >= n_q && append) {
      // key block layout [d/32][16][32]: dim i of this token at (i / 32, off, i % 32)
      const int g = head - n_q;
      bf16* kb = kpool + ((size_t)blk * n_kv + g) * (kBlock * d) + off * 32;
      *reinterpret_cast<bf16x8*>(kb + (i0 >> 5) * (kBlock * 32) + (i0 & 31)) = o1;
      *reinterpret_cast<bf16x8*>(kb + ((i0 + half) >> 5) * (kBlock * 32) + ((i0 + half) & 31)) = o2;
    }
  }
  if (!append) return;
  // v element i = (head g, dim j) to row (g, j) of the block; consecutive threads take
  // consecutive i, so one store instruction touches 16 lines (rows are 32 bytes apart)
  const bf16* vrow = row + (n_q + n_kv) * d;
  bf16* vb = vpool + (size_t)blk * n_kv * d * kBlock + off;
  for (int i = threadIdx.x; i < n_kv * d; i += 256) vb[(size_t)i * kBlock] = vrow[i];
}

hipError_t launch_rope_kv(bf16* qkv, const int32_t* tok_pos, const int32_t* tok_slot, const float* inv_freq,
                          bf16* kpool, bf16* vpool, int t_begin, int t_end, int n_q, int n_kv, int d,
                          hipStream_t s, int t_defer) {
  if (t_end <= t_begin) return hipSuccess;
  hipLaunchKernelGGL(rope_kv_kernel, dim3(t_end - t_begin), dim3(256), 0, s, qkv, tok_pos, tok_slot, inv_freq,
                     kpool, vpool, t_begin, t_defer, n_q, n_kv, d);
  return hipGetLastError();
}

// The paged KV append of tokens whose rotated k and v are already in qkv: one wave per
// token, k rows in 16-byte pieces into the 32-dim column chunks; v dim-major, one 2-byte
// store per dimension row of the block, consecutive lanes on consecutive dimensions so
// that one store instruction touches 16 lines (dimension rows are 32 bytes apart) rather
// than one line per lane.
__global__ __launch_bounds__(256) void kv_append_kernel(const bf16* __restrict__ qkv,
                                                        const int32_t* __restrict__ tok_slot, bf16* __restrict__ kpool,
                                                        bf16* __restrict__ vpool, int t_begin, int t_end, int n_q,
                                                        int n_kv, int d) {
  const int t = t_begin + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= t_end) return;
  const int lane = threadIdx.x & 63;
  const int slot = tok_slot[t];
  const int blk = slot / kBlock, off = slot % kBlock;
  const bf16* row = qkv + (size_t)t * (n_q + 2 * n_kv) * d;
  const bf16* krow = row + n_q * d;
  const bf16* vrow = row + (n_q + n_kv) * d;
  const int pieces = n_kv * d / 8;  // 16-byte pieces of the token's k
  for (int c = lane; c < pieces; c += 64) {
    const int g = (c * 8) / d, j0 = (c * 8) % d;
    const bf16x8 k = *reinterpret_cast<const bf16x8*>(krow + c * 8);
    bf16* kb = kpool + ((size_t)blk * n_kv + g) * (kBlock * d) + off * 32;
    *reinterpret_cast<bf16x8*>(kb + (j0 >> 5) * (kBlock * 32) + (j0 & 31)) = k;
  }
  // v element i = (head g, dim j) goes to row (g, j) of the block: lanes take consecutive i
  bf16* vb = vpool + (size_t)blk * n_kv * d * kBlock + off;
  for (int i = lane; i < n_kv * d; i += 64) vb[(size_t)i * kBlock] = vrow[i];
}

hipError_t launch_kv_append(const bf16* qkv, const int32_t* tok_slot, bf16* kpool, bf16* vpool, int t_begin,
                            int t_end, int n_q, int n_kv, int d, hipStream_t s) {
  if (t_end <= t_begin) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3((t_end - t_begin + 3) / 4), dim3(256), 0, s, qkv, tok_slot, kpool, vpool,
                     t_begin, t_end, n_q, n_kv, d);
  return hipGetLastError();
}

}  // namespace nf
