// Internal declarations of libnanoflow: device vector types, kernel launchers and the
// context structure. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/nanoflow.h"
#include "nf_batch.h"

namespace nf {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlock = 16;       // KV block size (tokens)
constexpr int kMaxGroup = 16;    // max query heads per KV head (MFMA column count)
constexpr int kNumXcd = 8;       // XCDs of an MI355X

// Device helpers shared by the kernels that stream tiles into LDS with direct-to-LDS loads.

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier ordering LDS only. __syncthreads() (a workgroup fence) also waits for
// every outstanding global load, vmcnt(0), which would drain the slabs still in flight.
// Here: this wave's LDS reads complete (lgkmcnt(0)), then s_barrier; the empty asm
// statements keep the compiler from moving memory accesses across the barrier. Slab data
// written by the load unit is covered by the explicit vmcnt wait before the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------------
// kernel launchers (defined in the .hip files)
// ---------------------------------------------------------------------------------------

// Grouped products (one per expert): see launch_gemm_grouped. Passed by value to the
// pipelined GEMM kernel; unused by its plain instantiations.
struct GroupArgs {
  const int32_t* grp;     // device [2 n_groups]: rows of each group, first grouped row of each group
  const int32_t* a_rows;  // device, optional: A row of each grouped row (gather); null = contiguous
  int n_groups;
  long long b_stride;     // elements between consecutive groups' B matrices
};

struct GemmVariant {
  int bm, bn, bk, ks;  // tile, k step, K slices (split-K; 1 = none)
  int stages = 4;      // LDS slabs of the pipelined kernels
  int waves = 4;       // waves per workgroup (pipelined kernels: 4 or 8)
  int b_stages = 0;    // slabs of a separate B ring (0: A and B share the STAGES ring)
};
int gemm_variant_count();
GemmVariant gemm_variant(int i);
int gemm_default_variant(int m, int n, int k, int epilogue);
bool gemm_variant_supported(int v, int m, int n, int k, int epilogue);
// fp32 workspace a variant needs for an m x n product (split-K partials; 0 for most)
size_t gemm_workspace_bytes(int variant, int m, int n);
// C = A B^T (+ epilogue); returns hipError_t of the launch. ws: workspace of at least
// gemm_workspace_bytes(variant, m, n) bytes (may be null when that is 0).
hipError_t launch_gemm(const bf16* A, const bf16* B, bf16* C, const bf16* R, int m, int n, int k,
                       int epilogue, int variant, hipStream_t s, float* ws = nullptr, size_t ws_bytes = 0);
// Set the kernel attributes of every GEMM configuration (plain and grouped) up front, so
// that launches make no other runtime call. Launches nothing.
hipError_t gemm_prepare_kernels();

// C = A B_g^T per group g (epilogue 0 store or 2 SwiGLU), pipelined tiles (variants 6-9),
// k a multiple of 32, n of 8. grp: device [2 n_groups] (rows, first row in the grouped
// order); n_rows: total grouped rows (an upper bound on the sum of grp rows is enough).
// C rows follow the grouped order; A rows too unless a_rows gathers them.
hipError_t launch_gemm_grouped(const bf16* A, const int32_t* a_rows, const bf16* B, long long b_stride, bf16* C,
                               const int32_t* grp, int n_groups, int n_rows, int n, int k, int epilogue, int variant,
                               hipStream_t s);
bool gemm_grouped_variant_ok(int variant, int n, int k, int epilogue);
int gemm_grouped_default_variant(int n_rows, int n_groups, int k, int epilogue);

// MoE: router + dispatch of tokens [t_begin, t_end) (sel/wts/pos/src indexed by token
// entry 2 t + k; grp: this nano-batch's [2 n_experts] group table), and the combine.
hipError_t launch_moe_route(const bf16* h2, const bf16* wr, int t_begin, int t_end, int H, int n_experts, int32_t* sel,
                            float* wts, int32_t* pos, int32_t* src, int32_t* grp, hipStream_t s);
hipError_t launch_moe_combine(const bf16* x1, const bf16* out, const int32_t* pos, const float* wts, bf16* y,
                              int t_begin, int t_end, int H, hipStream_t s);

// Move the K/V of the listed (block, token run) items between a pool and token-major
// staging rows (to_pool: staging -> pool). d in {64, 128}.
hipError_t launch_kv_move(bool to_pool, bf16* kpool, bf16* vpool, bf16* stage, const KvMoveItem* items, int n_items,
                          int n_kv, int d, hipStream_t s);

hipError_t launch_rmsnorm(const bf16* x, const bf16* g, bf16* out, int m, int n, float eps,
                          hipStream_t s);

// Rotary embedding of q and k (both in place in qkv) and the paged KV append of tokens
// [max(t_begin, t_defer), t_end); tokens below t_defer are appended later by launch_kv_append.
hipError_t launch_rope_kv(bf16* qkv, const int32_t* tok_pos, const int32_t* tok_slot,
                          const float* inv_freq, bf16* kpool, bf16* vpool, int t_begin, int t_end,
                          int n_q, int n_kv, int d, hipStream_t s, int t_defer = 0);
hipError_t launch_kv_append(const bf16* qkv, const int32_t* tok_slot, bf16* kpool, bf16* vpool, int t_begin,
                            int t_end, int n_q, int n_kv, int d, hipStream_t s);

// ev_start / ev_stop: optional timing events recorded by the dispatch itself (both or none).
// new_from_qkv: each request's newest key (position n_keys - 1) comes from its qkv row (rotated
// k, v) instead of the pool, which then need not hold it yet.
hipError_t launch_decode_attn(const bf16* qkv, const bf16* kpool, const bf16* vpool,
                              const int32_t* block_table, int max_blocks, const DecodeItem* items,
                              int n_items, float* part_o, float* part_ml, bf16* out, int n_q,
                              int n_kv, int d, int max_grid, int nb, int ring, hipStream_t s,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                              int new_from_qkv = 0);
bool decode_config_supported(int nb, int ring);
hipError_t launch_decode_combine(const CombineItem* combines, int n_combines, const float* part_o,
                                 const float* part_ml, bf16* out, int n_q, int n_kv, int d,
                                 hipStream_t s);

// Prefill attention of the listed items, then the merge of the split tiles' partials
// (combines: one per query of a split tile; partial slots as in PrefillItem).
hipError_t launch_prefill_attn(const bf16* qkv, const bf16* kpool, const bf16* vpool,
                               const int32_t* block_table, int max_blocks, const PrefillItem* items,
                               int n_items, const CombineItem* combines, int n_combines, float* part_o,
                               float* part_ml, bf16* out, int n_q, int n_kv, int d, hipStream_t s);

}  // namespace nf
