// Mixture-of-experts FFN pieces (summary page, "MoE models": an extra gate-routing
// operation, and the FFN as a grouped GEMM where different experts compute on different
// tokens):
//  - moe_router_kernel: per token, the router logits (fp32 dot products of the bf16 h2 row
//    with each expert's router row), the two largest (ties go to the lower expert index)
//    and their softmax weights;
//  - moe_dispatch_kernel: a stable counting sort of the (token, choice) entries of one
//    nano-batch by expert: each entry's row in the grouped order, the token of every
//    grouped row, and per expert its row count and first grouped row;
//  - moe_combine_kernel: y = x1 + w0 * out[row of choice 0] + w1 * out[row of choice 1],
//    summed in fp32 and rounded once.
// The expert products themselves run as grouped GEMMs (launch_gemm_grouped).
#include "nf_internal.h"

namespace nf {

// One wave per token, four tokens per workgroup.
template <int E>
__global__ __launch_bounds__(256) void moe_router_kernel(const bf16* __restrict__ h2, const bf16* __restrict__ wr,
                                                        int t_begin, int t_end, int H, int32_t* __restrict__ sel,
                                                        float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = t_begin + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= t_end) return;
  const bf16* x = h2 + (size_t)t * H;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  for (int c = lane * 8; c < H; c += 64 * 8) {
    const bf16x8 xv = *reinterpret_cast<const bf16x8*>(x + c);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wr + (size_t)e * H + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[e] += (float)xv[i] * (float)wv[i];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[e] += __shfl_xor(acc[e], off);
  // the two largest logits; a strict comparison keeps the lower index on ties
  int e0 = 0;
  float l0 = acc[0];
#pragma unroll
  for (int e = 1; e < E; ++e)
    if (acc[e] > l0) {
      l0 = acc[e];
      e0 = e;
    }
  int e1 = e0 == 0 ? 1 : 0;
  float l1 = acc[e1];
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e != e0 && acc[e] > l1) {
      l1 = acc[e];
      e1 = e;
    }
  if (lane == 0) {
    // softmax over the two chosen logits: d = exp(l1 - l0) in (0, 1]
    const float d = __expf(l1 - l0);
    sel[2 * t] = e0;
    sel[2 * t + 1] = e1;
    wts[2 * t] = 1.0f / (1.0f + d);
    wts[2 * t + 1] = d / (1.0f + d);
  }
}

// One workgroup per nano-batch [t_begin, t_end): entries i = 2 (t - t_begin) + k. Thread j
// sorts a contiguous run of entries; runs are ranked by a per-expert scan across threads,
// so grouped rows keep entry order within each expert (deterministic).
template <int E>
__global__ __launch_bounds__(256) void moe_dispatch_kernel(const int32_t* __restrict__ sel, int t_begin, int t_end,
                                                          int32_t* __restrict__ pos, int32_t* __restrict__ src,
                                                          int32_t* __restrict__ grp) {
  __shared__ int32_t cnt[256][E];
  __shared__ int32_t tot[E];
  __shared__ int32_t first[E];
  const int tid = threadIdx.x;
  const int n = 2 * (t_end - t_begin);
  const int per = (n + 255) / 256;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  const int32_t* s = sel + 2 * t_begin;
  int c[E];
#pragma unroll
  for (int e = 0; e < E; ++e) c[e] = 0;
  for (int i = i0; i < i1; ++i) {
    const int e = s[i];
#pragma unroll
    for (int x = 0; x < E; ++x) c[x] += (x == e);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) cnt[tid][e] = c[e];
  __syncthreads();
  if (tid < E) {  // exclusive scan of expert tid over the threads' runs
    int run = 0;
    for (int j = 0; j < 256; ++j) {
      const int v = cnt[j][tid];
      cnt[j][tid] = run;
      run += v;
    }
    tot[tid] = run;
    grp[tid] = run;  // rows of expert tid
  }
  __syncthreads();
  if (tid == 0) {
    int r = 0;
    for (int e = 0; e < E; ++e) {
      first[e] = r;
      grp[E + e] = r;
      r += tot[e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) c[e] = first[e] + cnt[tid][e];
  for (int i = i0; i < i1; ++i) {
    const int e = s[i];
    int p = 0;
#pragma unroll
    for (int x = 0; x < E; ++x)
      if (x == e) p = c[x]++;
    pos[2 * t_begin + i] = p;
    src[2 * t_begin + p] = t_begin + i / 2;
  }
}

// One workgroup per token row; 8 columns per thread and step.
__global__ __launch_bounds__(256) void moe_combine_kernel(const bf16* __restrict__ x1, const bf16* __restrict__ out,
                                                         const int32_t* __restrict__ pos, const float* __restrict__ wts,
                                                         bf16* __restrict__ y, int t_begin, int H) {
  const int t = t_begin + blockIdx.x;
  const int p0 = pos[2 * t], p1 = pos[2 * t + 1];  // rows of this nano-batch's grouped output
  const float w0 = wts[2 * t], w1 = wts[2 * t + 1];
  const bf16* o0 = out + ((size_t)2 * t_begin + p0) * H;
  const bf16* o1 = out + ((size_t)2 * t_begin + p1) * H;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(x1 + (size_t)t * H + c);
    const bf16x8 u = *reinterpret_cast<const bf16x8*>(o0 + c);
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(o1 + c);
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)((float)a[i] + w0 * (float)u[i] + w1 * (float)v[i]);
    *reinterpret_cast<bf16x8*>(y + (size_t)t * H + c) = r;
  }
}

bool moe_experts_supported(int n_experts) { return n_experts == 4 || n_experts == 8 || n_experts == 16; }

hipError_t launch_moe_route(const bf16* h2, const bf16* wr, int t_begin, int t_end, int H, int n_experts, int32_t* sel,
                            float* wts, int32_t* pos, int32_t* src, int32_t* grp, hipStream_t s) {
  if (t_end <= t_begin) return hipSuccess;
  const int grid = (t_end - t_begin + 3) / 4;
#define NF_MOE_CASE(EE)                                                                                          \
  case EE:                                                                                                       \
    hipLaunchKernelGGL(moe_router_kernel<EE>, dim3(grid), dim3(256), 0, s, h2, wr, t_begin, t_end, H, sel, wts); \
    hipLaunchKernelGGL(moe_dispatch_kernel<EE>, dim3(1), dim3(256), 0, s, sel, t_begin, t_end, pos, src, grp);   \
    break;
  switch (n_experts) {
    NF_MOE_CASE(4)
    NF_MOE_CASE(8)
    NF_MOE_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef NF_MOE_CASE
  return hipGetLastError();
}

hipError_t launch_moe_combine(const bf16* x1, const bf16* out, const int32_t* pos, const float* wts, bf16* y,
                              int t_begin, int t_end, int H, hipStream_t s) {
  if (t_end <= t_begin) return hipSuccess;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(t_end - t_begin), dim3(256), 0, s, x1, out, pos, wts, y, t_begin, H);
  return hipGetLastError();
}

}  // namespace nf
