// KV-cache movement between a paged pool and token-major staging rows (summary page,
// "KV-cache management and offloading": tokens' K/V are copied out to host memory; for a
// follow-up round they are loaded back by one contiguous host-to-device copy and a
// GPU-side scatter into the fragmented pages).
//
// One workgroup per (run of tokens in one block, KV head). Staging row t holds a token's
// K [n_kv][d] then V [n_kv][d]. In the pool a (block, head) holds K as [d/32][16][32]
// (32-dim column chunks, each token-major) and V as [d][16] (dim-major): K moves in
// 16-byte pieces on both sides; V goes through an LDS tile [16][d] so that both the
// staging rows and the pool's 16-token rows are read and written whole.
#include "nf_internal.h"

namespace nf {

template <bool TO_POOL>
__global__ __launch_bounds__(256) void kv_move_kernel(bf16* __restrict__ kpool, bf16* __restrict__ vpool,
                                                      bf16* __restrict__ stage, const KvMoveItem* __restrict__ items,
                                                      int n_kv, int d) {
  __shared__ __align__(16) bf16 tile[kBlock * 128];
  const KvMoveItem it = items[blockIdx.x];
  const int g = blockIdx.y;
  const int nt = it.tok1 - it.tok0;
  const size_t row = (size_t)2 * n_kv * d;  // staging elements per token
  bf16* kb = kpool + ((size_t)it.blk * n_kv + g) * kBlock * d;
  bf16* vb = vpool + ((size_t)it.blk * n_kv + g) * d * kBlock;
  bf16* sk = stage + (size_t)it.row * row + (size_t)g * d;
  bf16* sv = stage + (size_t)it.row * row + (size_t)(n_kv + g) * d;
  const int v8 = d / 8;  // 16-byte pieces per head row
  // K: piece (t, c) = dims 8c .. 8c + 7 of token t
  for (int e = threadIdx.x; e < nt * v8; e += 256) {
    const int t = e / v8, j = (e % v8) * 8;
    bf16x8* p = reinterpret_cast<bf16x8*>(kb + (j >> 5) * (kBlock * 32) + (it.tok0 + t) * 32 + (j & 31));
    bf16x8* q = reinterpret_cast<bf16x8*>(sk + (size_t)t * row + j);
    if (TO_POOL)
      *p = *q;
    else
      *q = *p;
  }
  // V through the LDS tile [t][j]
  if (TO_POOL) {
    for (int e = threadIdx.x; e < nt * v8; e += 256) {
      const int t = e / v8, j = (e % v8) * 8;
      *reinterpret_cast<bf16x8*>(tile + t * d + j) = *reinterpret_cast<const bf16x8*>(sv + (size_t)t * row + j);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nt * d; e += 256) {
      const int j = e / nt, t = e % nt;
      vb[j * kBlock + it.tok0 + t] = tile[t * d + j];
    }
  } else {
    for (int e = threadIdx.x; e < nt * d; e += 256) {
      const int j = e / nt, t = e % nt;
      tile[t * d + j] = vb[j * kBlock + it.tok0 + t];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nt * v8; e += 256) {
      const int t = e / v8, j = (e % v8) * 8;
      *reinterpret_cast<bf16x8*>(sv + (size_t)t * row + j) = *reinterpret_cast<const bf16x8*>(tile + t * d + j);
    }
  }
}

hipError_t launch_kv_move(bool to_pool, bf16* kpool, bf16* vpool, bf16* stage, const KvMoveItem* items, int n_items,
                          int n_kv, int d, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (d > 128 || d % 32) return hipErrorInvalidValue;
  if (to_pool)
    hipLaunchKernelGGL(kv_move_kernel<true>, dim3(n_items, n_kv), dim3(256), 0, s, kpool, vpool, stage, items, n_kv, d);
  else
    hipLaunchKernelGGL(kv_move_kernel<false>, dim3(n_items, n_kv), dim3(256), 0, s, kpool, vpool, stage, items, n_kv,
                       d);
  return hipGetLastError();
}

}  // namespace nf
