/*
 * nanoflow.h — C ABI of libnanoflow: one nano-batched decoder-layer iteration on one
 * MI355X (gfx950), plus the per-operation entry points, the profiler and the pipeline search.
 *
 * The layer (following NanoFlow, arXiv 2408.12757; summary page sections "The
 * Intra-Device Parallelism Mechanism", "Auto-Search Stage I/II" and "The NanoFlow Runtime
 * System"; slides "8B Pipeline Design" and "Batch Formation"):
 *
 *   h   = RMSNorm(x) * g_attn
 *   qkv = h W_qkv^T ;  q, k <- rotary(q, k, position)      (KQV generation)
 *   pool[slot(token)] <- k, v                                (paged KV append)
 *   o   = causal GQA attention per request over the pool     (decode / prefill attention)
 *   x1  = x + o W_o^T                                         (O projection)
 *   h2  = RMSNorm(x1) * g_ffn
 *   a   = silu(h2 W_gate^T) * (h2 W_up^T)                     (Up/Gate)
 *   y   = x1 + a W_down^T                                      (Down)
 *
 * over a dense batch of decode requests (one new token each) followed by prefill chunks.
 * The batch is split into nano-batches of consecutive tokens; each operation runs as one
 * nano-operation per nano-batch, and nano-operations of different resource classes run
 * concurrently on CU-masked HIP streams ordered by events. A nano-operation depends on
 * another iff their parent operations are dependent and their token ranges intersect
 * (summary page, "Auto-Search Stage I", constraints on dependencies).
 *
 * Conventions
 *  - Every function returns nf_status: NF_OK (0) or a negative error code. No exception or
 *    abort crosses the ABI. nf_last_error(ctx) gives a text for the last failure.
 *  - Validation happens on the host before anything is enqueued: a failed call leaves
 *    device memory untouched.
 *  - "device" pointers are HIP device memory owned by the caller; "host" pointers are read
 *    during the call only (their contents are copied), so they may be reused on return.
 *  - Tensors are bfloat16 (bit patterns, round-to-nearest-even on every store) unless
 *    stated otherwise, row-major, densely packed.
 *  - Calls are asynchronous with respect to the host and ordered with respect to the
 *    stream argument; calls that share one nf_ctx must be ordered (same stream, or
 *    externally synchronized). One nf_ctx per host thread.
 *  - Departures from a plain reading of the problem statement, by design: the KV pool keeps
 *    keys in 32-dim column chunks and values dim-major inside a block (see nf_kv_pool), not
 *    token-major [block][kv head][16][d], because the attention kernels then read whole
 *    128-byte lines straight into matrix-core operands; and a plan lists its
 *    nano-operations as (kind, nano-batch, stream) triples in issue order (see nf_plan)
 *    instead of a separate op order and op-to-stream map, so one array fixes both.
 */
#ifndef NANOFLOW_H
#define NANOFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nf_status;

enum {
  NF_OK = 0,
  NF_E_ARG = -1,               /* null pointer, non-positive size, unsupported shape          */
  NF_E_BLOCK_RANGE = -2,       /* block id outside [0, num_blocks)                             */
  NF_E_BLOCK_TABLE_SHORT = -3, /* a request needs more blocks than its table row holds         */
  NF_E_SLOT_ALIAS = -4,        /* two new tokens would write the same KV slot                  */
  NF_E_PLAN = -5,              /* plan bounds / op list invalid, or its order deadlocks        */
  NF_E_CU_MASK = -6,           /* CU mask empty, or leaving an XCD without CUs                 */
  NF_E_HIP = -7,               /* a HIP runtime call failed                                    */
  NF_E_UNSUPPORTED = -8,       /* shape outside what the kernels implement                     */
  NF_E_CAPACITY = -9,          /* batch larger than the context's workspace limits             */
  NF_E_IO = -10                /* profile / plan file could not be read or written            */
};

/* CU masks cover the 256 CUs of an MI355X as 8 words of 32 bits. Bit i selects a CU of
 * XCD (i mod 8); a mask must give every XCD the same, non-zero number of CUs. */
#define NF_CU_MASK_WORDS 8

typedef struct nf_ctx nf_ctx;  /* owns streams, events, metadata workspace, split-KV scratch */

/* Layer shape. Supported: head_dim in {64, 128}; n_q_heads a multiple of n_kv_heads with
 * n_q_heads / n_kv_heads <= 16; block_size 16; hidden, ffn and n_q_heads*head_dim multiples
 * of 8. rms_eps and rope_base as in the model (1e-5 and 10000 for the LLaMA shapes).
 * n_experts = 0: dense SwiGLU FFN. n_experts > 0: mixture-of-experts FFN (summary page,
 * "MoE models": a gate-routing operation, then the experts as a grouped GEMM): router
 * logits h2 W_router^T, the top_k largest per token (ties: lower expert index), weights =
 * softmax over the chosen logits, FFN output = sum over the chosen experts of weight x
 * expert SwiGLU FFN of h2. Supported: n_experts in {4, 8, 16}, top_k = 2, hidden and ffn
 * multiples of 32. */
typedef struct {
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, ffn, block_size;
  float rms_eps, rope_base;
  int32_t n_experts; /* 0 = dense FFN                                                   */
  int32_t top_k;     /* experts per token (MoE only)                                     */
} nf_layer_cfg;

/* Weights, device, Linear layout [out, in]:
 *   g_attn [hidden], g_ffn [hidden]                     RMSNorm gains
 *   w_qkv  [(n_q + 2 n_kv) head_dim, hidden]            rows = q heads | k heads | v heads
 *   w_o    [hidden, n_q head_dim]
 *   w_gate_up [2 ffn, hidden]                           rows = gate (ffn) | up (ffn)
 *   w_down [hidden, ffn]
 * MoE layers (n_experts = E > 0): w_gate_up [E][2 ffn, hidden] and w_down [E][hidden, ffn]
 * (expert-major, each expert as above), w_router [E, hidden]; NULL for dense layers.      */
typedef struct {
  const void *g_attn, *w_qkv, *w_o, *g_ffn, *w_gate_up, *w_down;
  const void *w_router;
} nf_layer_weights;

/* Dense batch (slides, "Batch Formation": decode requests first, then prefill chunks).
 * Request r < n_decode is a decode request: one new token at position decode_ctx_len[r],
 * after decode_ctx_len[r] cached tokens. Request n_decode + j is a prefill chunk of
 * prefill_len[j] >= 1 new tokens at positions prefill_prefix_len[j] + i (prefix NULL = 0).
 * Tokens are laid out in request order; T = n_decode + sum(prefill_len).
 * block_table (host, [n_decode + n_prefill][max_blocks], int32) maps logical block b of a
 * request to its physical block ("LLM Inference Performance", PagedAttention; entries
 * unused by a request are ignored, -1 by convention). block_table_dev is an optional device
 * copy of the same table; when NULL the library uploads the host table each call.      */
typedef struct {
  int32_t n_decode;
  const int32_t *decode_ctx_len;     /* host [n_decode], >= 0                        */
  int32_t n_prefill;
  const int32_t *prefill_len;        /* host [n_prefill], >= 1                        */
  const int32_t *prefill_prefix_len; /* host [n_prefill] or NULL                      */
  const int32_t *block_table;        /* host [n_req][max_blocks]                       */
  int32_t max_blocks;
  const int32_t *block_table_dev;    /* device copy or NULL                           */
} nf_batch_desc;

/* Paged KV pool of one layer, device, caller-owned:
 *   k [num_blocks][n_kv][head_dim / 32][block_size][32]   within a block, the key dims in
 *                                                      column chunks of 32, each chunk
 *                                                      token-major (dim = chunk * 32 + j)
 *   v [num_blocks][n_kv][head_dim][block_size]         dim-major within a block
 * Position p of request r lives in block table[r][p / block_size] at offset
 * p % block_size. nf_layer_forward writes exactly the slots of this iteration's tokens.
 * (The chunked key layout makes one load instruction of the attention kernels cover whole
 * 128-byte lines: 16 tokens x 64 bytes of one chunk are contiguous.)                       */
typedef struct {
  void *k, *v;
  int32_t num_blocks;
} nf_kv_pool;

/* Nano-operation kinds of the layer (slides, "8B Pipeline Design": KQV, decode attention,
 * prefill attention, O, Up/Gate/Down). Norms, rotary and KV append ride in the dense ops. */
enum {
  NF_OP_KQV = 0,     /* RMSNorm_1 + KQV GEMM + rotary + KV append, rows of the nano-batch     */
  NF_OP_DECATTN = 1, /* decode attention of the decode requests in the nano-batch             */
  NF_OP_PFATTN = 2,  /* prefill attention of the prefill chunks whose last token is here      */
  NF_OP_O = 3,       /* O GEMM + residual, rows of the nano-batch                              */
  NF_OP_UGD = 4,     /* RMSNorm_2 + Up/Gate GEMM + SwiGLU + Down GEMM + residual               */
  NF_OP_KINDS = 5
};

/* Nano-batch plan. bounds[0] = 0 < bounds[1] < ... < bounds[n_nano] = T (token offsets).
 * Streams: n_streams (1..3) CU-masked streams; cu_masks holds n_streams * NF_CU_MASK_WORDS
 * words (NULL = every stream uses the whole GPU). Nano-operations: n_ops entries given in
 * issue order, each (op_kind, op_nano, op_stream); every (kind, nano) pair appears exactly
 * once. A stream runs its nano-operations in the listed order; cross-stream order follows
 * the range-intersection dependencies. A NULL plan runs one nano-batch sequentially on
 * the caller's stream (the non-overlapped baseline). decode_max_workgroups bounds the
 * decode-attention grid (its waves then stride over the work), i.e. the memory nano-op's
 * share of the CUs' wave slots when it shares them with the GEMMs.
 * op_lane (optional, NULL = each op's lane is its stream; else n_ops entries in 0..2)
 * groups nano-operations into lanes that run one op at a time in the listed order even
 * when their ops sit on different streams: a compute lane can then put some dense ops on a
 * CU-masked stream beside the memory stream and others on an unmasked stream, i.e. give
 * each nano-operation its own resource share (NanoFlow summary page, "Auto-Search Stage
 * II: Refining the Pipeline"), without two of its ops running at once.                     */
typedef struct {
  int32_t n_nano;
  const int32_t *bounds;
  int32_t n_streams;
  const uint32_t *cu_masks;
  int32_t n_ops;
  const int32_t *op_kind, *op_nano, *op_stream;
  int32_t decode_max_workgroups; /* cap on decode-attention workgroups, 0 = context default */
  const int32_t *op_lane;        /* NULL, or the lane (0..2) of each listed op              */
} nf_plan;

/* ---- context ---------------------------------------------------------------------------- */

/* Create a context on HIP device `device`: default kernel variants, no streams yet (masked
 * streams are created on first use and cached). Errors: NF_E_ARG, NF_E_HIP.                */
nf_status nf_ctx_create(int device, nf_ctx **out);
void nf_ctx_destroy(nf_ctx *ctx);
const char *nf_last_error(const nf_ctx *ctx);
/* Library version string, e.g. "nanoflow-mi355x 0.1". Never NULL. */
const char *nf_version(void);

/* Context tuning knobs (profiling, sweeps and tests; the defaults are the library's choice).
 * Each applies to later calls of the context only; results do not depend on them beyond
 * floating-point summation order. */

/* Decode split-KV chunk, in KV blocks per work item: 0 (default) = chosen per nano-op from
 * its work, else 1..4096. Errors: NF_E_ARG.                                                 */
nf_status nf_ctx_set_decode_split(nf_ctx *ctx, int32_t blocks);
/* Prefill attention work item: keys of a query tile per item, 0 (default) = chosen per
 * nano-op (the longest of 1024, 512, 256, 128 that still gives a workgroup per CU),
 * else a multiple of 32 up to 1024; a tile with more keys is split into items whose fp32
 * partials are merged after. Errors: NF_E_ARG.                                              */
nf_status nf_ctx_set_prefill_chunk(nf_ctx *ctx, int32_t keys);
/* Decode-attention launch: max_workgroups caps its grid (0 = one workgroup per four work
 * units; a smaller grid makes the kernel persistent, each wave looping over units), nbuf KV
 * blocks per online-softmax step and ring register buffers of nbuf blocks (ring - 1 steps in
 * flight). Supported (nbuf, ring): (0, 0) = chosen per launch (the default: (1, 2), or (2, 2)
 * when the launch has fewer waves than one round of (1, 2)'s wave slots), (1, 2..4),
 * (2, 2..3). Errors: NF_E_ARG.                                                               */
nf_status nf_ctx_set_decode_launch(nf_ctx *ctx, int32_t max_workgroups, int32_t nbuf, int32_t ring);
/* GEMM tile configuration of a dense op kind (NF_OP_KQV, NF_OP_O, NF_OP_UGD): which = 0 its
 * GEMM (Up/Gate for UGD), 1 the Down GEMM of UGD; variant -1 restores the library choice,
 * else an index of nf_gemm_variants. A variant not available at a call's shape or epilogue
 * falls back to the library choice there. Errors: NF_E_ARG.                                 */
nf_status nf_ctx_set_gemm_variant(nf_ctx *ctx, int32_t kind, int32_t which, int32_t variant);
/* Counters of the stack's graph path: captures made and replays launched since the context
 * was created (both stay 0 while graph replay is switched off). Errors: NF_E_ARG.          */
nf_status nf_ctx_graph_stats(nf_ctx *ctx, int64_t *captures, int64_t *launches);

/* ---- host-only helpers (no GPU needed) ------------------------------------------------------ */

/* Validate a batch against a shape and a pool size, and derive each token's position and
 * KV slot (slot = block * block_size + offset). pos_out / slot_out: host [T] or NULL.
 * Returns the first error found: NF_E_ARG (bad lengths), NF_E_BLOCK_TABLE_SHORT,
 * NF_E_BLOCK_RANGE, NF_E_SLOT_ALIAS. err_msg (host, err_cap bytes, may be NULL) receives
 * a description.                                                                          */
nf_status nf_batch_slots(const nf_layer_cfg *cfg, const nf_batch_desc *batch, int32_t num_blocks,
                         int32_t *pos_out, int32_t *slot_out, char *err_msg, size_t err_cap);

/* Dependency edges of a plan's nano-operations by range intersection. The edge list holds
 * pairs (i, j): op j (index into the plan's op list) depends on op i. Capacity cap pairs;
 * *n_edges receives the count (NF_E_CAPACITY if it exceeds cap). Also checks the plan:
 * NF_E_PLAN when bounds or the op list are invalid, or when per-stream order plus
 * dependencies contain a cycle. order_out (host [n_ops] or NULL) receives a global issue
 * order consistent with both.                                                              */
nf_status nf_plan_dependencies(const nf_batch_desc *batch, const nf_plan *plan, int32_t *edges,
                               int32_t cap, int32_t *n_edges, int32_t *order_out, char *err_msg,
                               size_t err_cap);

/* Flags of the layer-stack entry points. */
enum {
  NF_STACK_PIPELINE = 1, /* cross-layer nano-batch pipelining (see nf_stack_forward)          */
  NF_STACK_GRAPH = 2     /* replay a captured HIP graph of the stack (switched off: see below) */
};

/* Dependency edges and issue order of n_layers layers over one batch, each with `plan`
 * (see nf_stack_forward). Stack op l * n_ops + i is the plan's op i (plan order; the NULL
 * plan lists KQV, decode attention, prefill attention, O, UGD) in layer l. Edges (i, j):
 * op j depends on op i. listing_out (host [n_layers * n_ops] or NULL) receives the order in
 * which each stream takes its ops (every stream runs its ops in this order); order_out
 * (same size or NULL) a global issue order consistent with both. Errors as
 * nf_plan_dependencies; NF_E_ARG for n_layers < 1 or unknown flags.                         */
nf_status nf_stack_dependencies(const nf_batch_desc *batch, const nf_plan *plan, int32_t n_layers,
                                int32_t flags, int32_t *edges, int32_t cap, int32_t *n_edges,
                                int32_t *listing_out, int32_t *order_out, char *err_msg,
                                size_t err_cap);

/* ---- KV-cache offload and multi-round reload ---------------------------------------------- */

/* Token ranges of requests in a pool, for moving their K/V between the pool and host memory
 * (summary page, "KV-cache management and offloading"): request r's tokens at positions
 * first[r] .. first[r] + n_tokens[r] - 1, addressed through row r of block_table as in
 * nf_batch_desc. Host data is token-major: the ranges in request order, each token's K then
 * V, each [n_kv][head_dim] bf16 (2 n_kv head_dim values, 4 KB for the 8B shape).          */
typedef struct {
  int32_t n_req;
  const int32_t *first;       /* host [n_req], >= 0                                        */
  const int32_t *n_tokens;    /* host [n_req], >= 0                                        */
  const int32_t *block_table; /* host [n_req][max_blocks]                                  */
  int32_t max_blocks;
} nf_kv_ranges;

/* Offload: copy the ranges' K/V from `pool` to host_dst (host, sum(n_tokens) x 2 n_kv
 * head_dim bf16; pinned memory keeps the copy asynchronous): a gather kernel packs them
 * token-major into a context buffer, then one device-to-host copy (copy engine) — the
 * pages copy each token's KV out as it is produced, by the copy engine. host_dst is
 * complete when `stream` passes the copy. The pool is not modified. KV moves use buffers of
 * their own in the context: they may run on another stream than the context's layer calls
 * (e.g. beside the next layer, as the pages schedule their copies), but KV moves of one
 * context must be ordered among themselves.
 * Errors: NF_E_ARG, NF_E_BLOCK_RANGE, NF_E_BLOCK_TABLE_SHORT, NF_E_HIP.                   */
nf_status nf_kv_offload(nf_ctx *ctx, const nf_layer_cfg *cfg, const nf_kv_pool *pool,
                        const nf_kv_ranges *ranges, void *host_dst, void *stream);

/* Reload (multi-round conversations): write host_src (the layout above) into the ranges'
 * slots of `pool`, in two stages as the pages describe for paged KV: one contiguous
 * host-to-device copy into a context buffer, then a scatter kernel that fills each (block,
 * KV head) of the ranges. Only the ranges' slots change. host_src must stay valid until
 * `stream` passes the copy. Errors: as nf_kv_offload, plus NF_E_SLOT_ALIAS when two tokens
 * of the ranges map to one slot.                                                            */
nf_status nf_kv_reload(nf_ctx *ctx, const nf_layer_cfg *cfg, nf_kv_pool *pool,
                       const nf_kv_ranges *ranges, const void *host_src, void *stream);

/* ---- the layer --------------------------------------------------------------------------- */

/* One decoder-layer iteration. x_in, y_out: device [T][hidden] (may alias: every row is
 * read before it is overwritten). Writes y and this iteration's KV slots; everything else
 * in the pool is left unchanged. Work is enqueued after all prior work on `stream` and
 * `stream` waits for all of it on return (fork/join through events).
 * Errors: NF_E_ARG, NF_E_UNSUPPORTED, NF_E_BLOCK_*, NF_E_SLOT_ALIAS, NF_E_PLAN,
 * NF_E_CU_MASK, NF_E_CAPACITY, NF_E_HIP.                                                    */
nf_status nf_layer_forward(nf_ctx *ctx, const nf_layer_cfg *cfg, const nf_layer_weights *w,
                           const void *x_in, void *y_out, const nf_batch_desc *batch,
                           nf_kv_pool *pool, const nf_plan *plan, void *stream);

/* n_layers decoder-layer iterations over one dense batch, end to end: the layers of one
 * model iteration (summary page, "The NanoFlow Runtime System"; slides "8B Pipeline
 * Design": the next layer's KQV of a nano-batch follows this layer's Down of the same
 * nano-batch). Layer l applies weights[l] to the output of layer l - 1 (layer 0 to x_in)
 * and appends to pools[l]; y_out receives the last layer's output. weights, pools: host
 * arrays [n_layers] of device tensors, laid out as for nf_layer_forward; every pool has
 * the same num_blocks and is addressed through the one block table of `batch` (one paged
 * KV cache per layer, one block allocation per request); pools must not overlap (distinct
 * k and v buffers per layer). x_in and y_out may alias; layers after the first run in
 * place on y_out. The batch is laid out and its metadata uploaded once for all layers.
 * plan: as for nf_layer_forward, applied to every layer.
 * flags: NF_STACK_PIPELINE — layer l + 1's KQV of a nano-batch is issued as soon as layer
 *   l's UGD ops it depends on (intersecting rows) are, instead of after all of layer l, so
 *   on a multi-stream plan the next layer's decode attention of nano-batch j can overlap
 *   this layer's dense ops of nano-batch j + 1 (results are identical).
 *   NF_STACK_GRAPH — capture the enqueued work once into a HIP graph owned by the context
 *   and replay it while the batch (contents included), plan, flags, weights, pools and
 *   x_in / y_out pointers are unchanged. Switched off in this build: a call with this flag
 *   returns NF_E_UNSUPPORTED before enqueueing anything.
 * Work is enqueued after all prior work on `stream` and `stream` waits for all of it.
 * Errors: as nf_layer_forward; NF_E_ARG for n_layers < 1, null arrays, unknown flags,
 * unequal num_blocks or overlapping pools; NF_E_UNSUPPORTED as above.                      */
nf_status nf_stack_forward(nf_ctx *ctx, const nf_layer_cfg *cfg, int32_t n_layers,
                           const nf_layer_weights *weights, const void *x_in, void *y_out,
                           const nf_batch_desc *batch, nf_kv_pool *pools, const nf_plan *plan,
                           int32_t flags, void *stream);

/* Intermediate buffers of the last nf_layer_forward call, for inspection (device pointers
 * into the context's workspace, valid until the next call): which = 0 h, 1 qkv (q rotated),
 * 2 attention output [T][n_q head_dim], 3 x1, 4 h2, 5 a [T][ffn]. Errors: NF_E_ARG.         */
nf_status nf_debug_buffer(nf_ctx *ctx, int32_t which, void **ptr, size_t *bytes);

/* ---- per-operation entry points (tests and profiler); one stream each --------------------
 *
 * Each operation of the layer runs alone on one stream, as the profiler needs it: the pages
 * time every operation type in isolation, for every batch size and kernel configuration,
 * to find its best interference-free time D_best (summary page, "Kernel Profiling and
 * Interference Modeling", interference-free kernel profiling). The layer call runs the
 * same kernels. Errors of every call: NF_E_ARG for null pointers or bad sizes (nothing is
 * enqueued), NF_E_UNSUPPORTED for a shape the kernels do not implement, NF_E_HIP when a
 * launch fails. */

/* The dense projections of the layer (summary page, "Operation classification": KQV, O,
 * Up/Gate and Down are the compute-bound GEMMs of a decoder layer; slides "8B Pipeline
 * Design"). C[m][n] = A[m][k] B[n][k]^T (+ epilogue), all device bf16, row-major:
 * A [m][k] activations, B [n][k] a Linear-layout weight. epilogue 0: store; 1: C = R + A B^T
 * (the residual add after O and Down) with R device [m][n] (may alias C); 2: SwiGLU
 * (silu(gate) * up of the FFN) — B holds 2n rows (gate | up) and
 * C[m][n] = silu(A Bg^T) * (A Bu^T). variant: -1 = library choice, else a tile
 * configuration index (see nf_gemm_variants). k and n multiples of 8. Split-K variants keep
 * their fp32 partials in a workspace the context owns (grown on demand).                   */
nf_status nf_op_gemm(nf_ctx *ctx, const void *A, const void *B, void *C, const void *R, int32_t m,
                     int32_t n, int32_t k, int32_t epilogue, int32_t variant, void *stream);
/* nf_op_gemm for callers that cannot allocate device memory: code under HIP-graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, result and errors
 * as nf_op_gemm, but the call allocates nothing: the fp32 partials of a split-K
 * configuration go to a static scratch array of 64 MiB per GPU (held until the process
 * ends) instead of the context's workspace. Every partial is written before it is read,
 * so nothing needs clearing. Calls on one GPU share that array: calls that overlap in time
 * on one GPU (different streams or contexts, not ordered) race. NF_E_CAPACITY when the
 * product's partials (K slices x m x n x 4 bytes) exceed 64 MiB; nothing is enqueued then. */
nf_status nf_op_gemm_noalloc(nf_ctx *ctx, const void *A, const void *B, void *C, const void *R,
                             int32_t m, int32_t n, int32_t k, int32_t epilogue, int32_t variant,
                             void *stream);
/* Number of GEMM tile configurations and, for index i, into out5: its tile (bm, bn), k
 * step, number of K slices (split-K, 1 = none; not with the SwiGLU epilogue) and waves per
 * workgroup (the SwiGLU epilogue needs each wave's bn / (waves / 2) columns to be a
 * multiple of 64). */
nf_status nf_gemm_variants(int32_t *count, int32_t index, int32_t *out5);
/* Host query, no device needed: the tile configuration nf_op_gemm (and the layer) takes
 * for variant -1 at this shape, and whether it is available there (*supported = 1). Same
 * argument rules as nf_op_gemm. Errors: NF_E_ARG (bad sizes or epilogue, NULL outputs),
 * NF_E_UNSUPPORTED (n or k not a multiple of 8).                                            */
nf_status nf_gemm_choice(int32_t m, int32_t n, int32_t k, int32_t epilogue, int32_t *variant,
                         int32_t *supported);

/* The norm before attention and before the FFN (the pages name no norm: a pre-norm LLaMA
 * layer's RMSNorm, eps from the model): out[r][:] = x[r] / sqrt(mean(x[r]^2) + eps) * g for
 * rows r in [0, m), width n (a multiple of 8). x, out device [m][n]; g device [n].          */
nf_status nf_op_rmsnorm(nf_ctx *ctx, const void *x, const void *g, void *out, int32_t m, int32_t n,
                        float eps, void *stream);

/* Rotary embedding of q and k and the paged KV append (slides, "Batch Formation": new
 * tokens' K/V go to their pages; "Inside nano-vLLM", the slot mapping locates each new KV
 * store): q and k of qkv (device [T][(n_q+2n_kv) d], both rotated in place) rotated at the
 * batch's token positions, then k and v written to each token's slot of the pool
 * (slot = table[r][pos / 16] * 16 + pos % 16). Only those slots change. Errors as the
 * layer call for the batch (NF_E_BLOCK_*, NF_E_SLOT_ALIAS).                                  */
nf_status nf_op_rope_kv_append(nf_ctx *ctx, const nf_layer_cfg *cfg, void *qkv,
                               const nf_batch_desc *batch, nf_kv_pool *pool, void *stream);

/* Decode attention, the memory-bound operation of the layer (summary page, "Operation
 * classification": decode attention loads each request's KV-cache): for every decode
 * request r and query head h, softmax(q k^T / sqrt(d)) v over the request's decode_ctx_len[r]
 * + 1 keys of KV head h / (n_q / n_kv), read through its block-table row. q is read from qkv
 * (device [T][(n_q+2n_kv) d], already rotated), K/V from the pool (already holding this
 * iteration's tokens); writes the decode rows of out (device [T][n_q d]) and nothing else.
 * kv_split_blocks: split-KV chunk in blocks, 0..4096 (0 = the context's default). The
 * split-KV partials live in the context's workspace. Errors as the layer call for the
 * batch.                                                                                     */
nf_status nf_op_decode_attn(nf_ctx *ctx, const nf_layer_cfg *cfg, const void *qkv,
                            const nf_batch_desc *batch, const nf_kv_pool *pool, void *out,
                            int32_t kv_split_blocks, void *stream);

/* Prefill attention, compute-bound, causal within each prefill chunk ("Inside nano-vLLM",
 * prefill batching keeps request boundaries; slides "Batch Formation"): query i of chunk j
 * attends to keys 0 .. prefill_prefix_len[j] + i of its request. Same buffers as
 * nf_op_decode_attn; writes the prefill rows of out only.                                   */
nf_status nf_op_prefill_attn(nf_ctx *ctx, const nf_layer_cfg *cfg, const void *qkv,
                             const nf_batch_desc *batch, const nf_kv_pool *pool, void *out,
                             void *stream);

/* The mixture-of-experts FFN alone (see nf_layer_cfg), for tests and profiling:
 * y = x1 + sum over the top_k chosen experts of weight x expert(h2), for n_tokens rows.
 * h2, x1, y: device [n_tokens][hidden] (y may alias x1); w: the layer's weights (g_* and
 * attention weights unused). sel_out (int32) and wts_out (float), device [n_tokens][top_k]
 * or NULL: the chosen experts (largest logit first) and their weights. Errors: NF_E_ARG,
 * NF_E_UNSUPPORTED (dense cfg or unsupported MoE shape), NF_E_HIP.                         */
nf_status nf_op_moe_ffn(nf_ctx *ctx, const nf_layer_cfg *cfg, const nf_layer_weights *w, const void *h2,
                        const void *x1, void *y, int32_t n_tokens, int32_t *sel_out, float *wts_out,
                        void *stream);

/* ---- kernel timing ------------------------------------------------------------------------ */

/* Kernel classes that can be timed. */
enum {
  NF_K_DECODE_ATTN = 0,    /* split-KV decode attention kernel              */
  NF_K_DECODE_COMBINE = 1, /* split-KV merge kernel                          */
  NF_K_PREFILL_ATTN = 2,   /* prefill attention kernel                       */
  NF_K_GEMM_KQV = 3,
  NF_K_GEMM_O = 4,
  NF_K_GEMM_UG = 5,        /* Up/Gate GEMM with the SwiGLU epilogue           */
  NF_K_GEMM_DOWN = 6,
  NF_K_RMSNORM = 7,
  NF_K_ROPE_KV = 8,
  NF_K_MOE_ROUTE = 9,      /* MoE router + dispatch (grouped GEMMs count as UG / Down) */
  NF_K_MOE_COMBINE = 10,   /* MoE weighted combine + residual                */
  NF_K_CLASSES = 11
};

/* Start collecting kernel timings for the classes whose bit is set in class_mask (0 stops):
 * every later launch of such a kernel by nf_layer_forward is bracketed by HIP timing events
 * recorded on the stream the kernel runs on (decode attention: by the kernel's dispatch
 * itself, so its timing adds no marker between it and its neighbours). Clears earlier
 * records. Errors: NF_E_ARG.                                                                */
nf_status nf_ctx_set_timing(nf_ctx *ctx, uint32_t class_mask);

/* Launch count and total / min / max duration (ms) of the recorded launches of class `cls`
 * since the last nf_ctx_set_timing. Waits for those launches to finish. min_ms / max_ms may
 * be NULL. Errors: NF_E_ARG, NF_E_HIP.                                                        */
nf_status nf_timing_summary(nf_ctx *ctx, int32_t cls, int32_t *count, double *total_ms, double *min_ms,
                            double *max_ms);

/* Plain device-to-device copy of `bytes` bytes (a multiple of 16; both pointers 16-byte
 * aligned; the ranges must not overlap), enqueued on `stream`: every lane moves 16 bytes per
 * load and store, loads nontemporal like the KV stream of decode attention. It reads and
 * writes exactly `bytes` bytes once, which makes it the known-size reference that scales
 * hardware traffic counters (bytes per counted unit). Errors: NF_E_ARG, NF_E_HIP.         */
nf_status nf_copy_reference(void *dst, const void *src, size_t bytes, void *stream);

/* ---- profiler and pipeline search (summary page, "Kernel Profiling and Interference
 *      Modeling"; "Auto-Search Stage I" and "Stage II") ----------------------------------- */

/* Interference-free profile: for each nano-operation kind and each batch size b in
 * step, 2 step, ..., max_tokens, time every kernel configuration on synthetic data shaped
 * like `batch_template` scaled to b tokens, keep the best (D_best), and write JSON to
 * out_json. Errors: NF_E_ARG, NF_E_IO, NF_E_HIP.                                             */
nf_status nf_profile_ops(nf_ctx *ctx, const nf_layer_cfg *cfg, const nf_batch_desc *batch_template,
                         int32_t num_blocks, int32_t step, int32_t max_tokens, const char *out_json);

/* Pairwise interference: for each CU share R of the non-GEMM kernel in r_grid (n_r values in
 * (0,1)), and for the shared GPU without masks (plain and with bounded attention grids),
 * run a GEMM nano-op on a mask of (1-R) of the CUs and a decode-attention nano-op on a mask
 * of R concurrently, and record each one's speed relative to its own best (P values). The
 * plain fields of an entry come from the Up/Gate/Down nano-op; the KQV and O nano-ops are
 * measured the same way (p_gemm_both_kind, p_mem_both_kind, p_gemm_alone_kind, keyed by
 * kind). Writes JSON to out_json. Errors: NF_E_ARG, NF_E_IO, NF_E_HIP, NF_E_CU_MASK.        */
nf_status nf_profile_interference(nf_ctx *ctx, const nf_layer_cfg *cfg,
                                  const nf_batch_desc *batch_template, int32_t num_blocks,
                                  const float *r_grid, int32_t n_r, const char *out_json);

/* Two-stage search. Stage I: over nano-batch counts 1..max_nano (sizes multiples of
 * `granularity` summing to T, no two ops of one class overlapping, no interference),
 * minimize the makespan of the list schedule built from the D_best table. Stage II: fix
 * that structure and choose the CU share R of the memory stream from the R->P table to
 * minimize the makespan with interference. Input JSON as written by the profilers. Writes
 * the plan as JSON into plan_json_out (host buffer, cap bytes). Errors: NF_E_ARG, NF_E_IO,
 * NF_E_CAPACITY, NF_E_PLAN.                                                                  */
nf_status nf_plan_search(const char *dbest_json, const char *rp_json, const nf_batch_desc *batch,
                         int32_t max_nano, int32_t granularity, char *plan_json_out, size_t cap);

#ifdef __cplusplus
}
#endif
#endif /* NANOFLOW_H */
