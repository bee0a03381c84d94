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

// One workgroup of 256 threads per row; each thread owns chunks of 8 contiguous elements.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const bf16* __restrict__ x, const bf16* __restrict__ g,
                                                      bf16* __restrict__ out, int n, float eps) {
  const int row = blockIdx.x;
  const bf16* xr = x + (size_t)row * n;
  bf16* orow = out + (size_t)row * n;
  const int chunks = n / 8;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = (float)v[j];
      ss += f * f;
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
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c * 8);
    const bf16x8 gv = *reinterpret_cast<const bf16x8*>(g + c * 8);
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (bf16)(((float)v[j] * inv) * (float)gv[j]);
    *reinterpret_cast<bf16x8*>(orow + c * 8) = o;
  }
}

hipError_t launch_rmsnorm(const bf16* x, const bf16* g, bf16* out, int m, int n, float eps, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(m), dim3(256), 0, s, x, g, out, n, eps);
  return hipGetLastError();
}

// One workgroup per token. Threads walk the (head, pair) space of q and k heads, then the
// v elements. q is rotated in place in qkv; k and v go to the pool.
__global__ __launch_bounds__(256) void rope_kv_kernel(bf16* __restrict__ qkv, const int32_t* __restrict__ tok_pos,
                                                      const int32_t* __restrict__ tok_slot,
                                                      const float* __restrict__ inv_freq, bf16* __restrict__ kpool,
                                                      bf16* __restrict__ vpool, int t_begin, int n_q, int n_kv,
                                                      int d) {
  const int t = t_begin + blockIdx.x;
  const int pos = tok_pos[t];
  const int slot = tok_slot[t];
  const int blk = slot / kBlock, off = slot % kBlock;
  const int half = d / 2;
  const int width = (n_q + 2 * n_kv) * d;
  bf16* row = qkv + (size_t)t * width;
  const float fpos = (float)pos;
  const int n_pairs = (n_q + n_kv) * half;
  for (int i = threadIdx.x; i < n_pairs; i += 256) {
    const int head = i / half, j = i % half;
    float sn, cs;
    sincosf(fpos * inv_freq[j], &sn, &cs);  // full-range reduction (angles reach ~4096 rad)
    bf16* hp = row + head * d;
    const float x1 = (float)hp[j], x2 = (float)hp[j + half];
    const bf16 o1 = (bf16)(x1 * cs - x2 * sn);
    const bf16 o2 = (bf16)(x2 * cs + x1 * sn);
    if (head < n_q) {
      hp[j] = o1;
      hp[j + half] = o2;
    } else {
      // key block layout [d/32][16][32]: dim i of this token at (i / 32, off, i % 32)
      const int g = head - n_q;
      bf16* kb = kpool + ((size_t)blk * n_kv + g) * (kBlock * d) + off * 32;
      kb[(j >> 5) * (kBlock * 32) + (j & 31)] = o1;
      kb[((j + half) >> 5) * (kBlock * 32) + ((j + half) & 31)] = o2;
    }
  }
  const bf16* vrow = row + (n_q + n_kv) * d;
  for (int i = threadIdx.x; i < n_kv * d; i += 256) {
    const int g = i / d, j = i % d;
    vpool[(((size_t)blk * n_kv + g) * d + j) * kBlock + off] = vrow[i];
  }
}

hipError_t launch_rope_kv(bf16* qkv, const int32_t* tok_pos, const int32_t* tok_slot, const float* inv_freq,
                          bf16* kpool, bf16* vpool, int t_begin, int t_end, int n_q, int n_kv, int d,
                          hipStream_t s) {
  if (t_end <= t_begin) return hipSuccess;
  hipLaunchKernelGGL(rope_kv_kernel, dim3(t_end - t_begin), dim3(256), 0, s, qkv, tok_pos, tok_slot, inv_freq,
                     kpool, vpool, t_begin, n_q, n_kv, d);
  return hipGetLastError();
}

}  // namespace nf
