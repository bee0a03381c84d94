// Host-side batch metadata and nano-operation DAG (no GPU calls). Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/nanoflow.h"

namespace nf {

// One decode split-KV work item: the blocks [blk_begin, blk_end) of request `req`
// (a decode request), for every KV head. `part` indexes the partial-result slots of the
// request (part_base + chunk) or is -1 when the request has a single chunk.
struct DecodeItem {
  int32_t req;        // request index (row of the block table)
  int32_t token;      // row of q / output
  int32_t n_keys;     // ctx + 1
  int32_t blk_begin;  // first logical block of this chunk
  int32_t blk_end;    // one past the last logical block
  int32_t part;       // partial slot index or -1
};

// One decode request that needs a split-KV combine.
struct CombineItem {
  int32_t token;
  int32_t part_begin;
  int32_t n_parts;
  int32_t pad;
};

// One prefill attention work item: a tile of consecutive queries of one prefill chunk
// (prefill_tile_queries of them) against a range of the request's keys. A tile whose keys
// are split over several items writes fp32 partials, merged by the decode combine kernel.
struct PrefillItem {
  int32_t req;        // request index (row of the block table)
  int32_t token0;     // dense-batch row of the first query of the request
  int32_t q_begin;    // first query (within the request) of this tile
  int32_t q_len;      // queries of the request
  int32_t prefix;     // cached prefix length
  int32_t key_begin;  // keys [key_begin, key_end) of the request: key_begin a multiple of
  int32_t key_end;    // 32, at most kPrefillMaxChunkKeys keys
  int32_t part;       // -1: the tile's only chunk (final output); else the partial slot of the
                      // tile's first query for this chunk (query i of the tile: part + i * n_chunks)
  int32_t n_chunks;   // chunks of the tile
  int32_t pad[3];
};

// Prefill attention workgroups: 4 waves of 32 queries each, covering heads_per_wg query
// heads of one KV group times 4 / heads_per_wg consecutive 32-query tiles (they share the
// KV tiles staged in LDS). A group of G query heads per KV head takes 4, 2 or 1 heads per
// workgroup, the largest that divides G.
inline int prefill_heads_per_wg(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }
inline int prefill_tile_queries(int G) { return 32 * (4 / prefill_heads_per_wg(G)); }
constexpr int kPrefillMaxChunkKeys = 1024;  // keys of one item: its <= 64 block ids fit one wave

// Prefill work of chunks (request r: q_len queries after prefix cached keys, rows from
// token0): tiles longest first, each tile's keys split into chunks of at most chunk_keys
// (a multiple of 32, <= kPrefillMaxChunkKeys). Items go to `items`; a split tile gets
// q_len-of-tile x n_chunks partial slots from n_parts on and one combine entry per query.
struct PrefillReq {
  int32_t req, token0, q_len, prefix;
};
void build_prefill_work(const std::vector<PrefillReq>& reqs, int n_q, int n_kv, int chunk_keys,
                        std::vector<PrefillItem>& items, std::vector<CombineItem>& comb, int32_t& n_parts);
// The chunk size build_work takes: the longest of 1024, 512, 256, 128 keys that gives at
// least kPrefillTargetWgs workgroups (128 when none does).
int prefill_chunk_keys(const std::vector<PrefillReq>& reqs, int n_q, int n_kv);
constexpr int kPrefillTargetWgs = 256;

// One request of the dense batch, in dense-batch order (decodes, then prefill chunks).
struct ReqInfo {
  int32_t t0, t1;    // token rows [t0, t1)
  int32_t cached;    // tokens already in the pool
  int32_t n_keys;    // cached + (t1 - t0)
  bool decode;
};

// Everything derived on the host from (cfg, batch, pool size), before any enqueue.
struct BatchLayout {
  int32_t T = 0;
  std::vector<ReqInfo> req;
  std::vector<int32_t> pos, slot;  // per token
};

// Validate and lay out a batch. Returns NF_OK or the first error, with a message.
nf_status build_layout(const nf_layer_cfg& cfg, const nf_batch_desc& b, int32_t num_blocks, BatchLayout& out,
                       std::string& err);

// Validate the layer shape against what the kernels implement.
nf_status check_cfg(const nf_layer_cfg& cfg, std::string& err);
// Expert counts the MoE kernels are built for (defined with them).
bool moe_experts_supported(int n_experts);

// A nano-operation of a plan with the token rows it reads/writes (its "range").
struct NanoOp {
  int32_t kind, nano, stream;
  // rows of the op: one interval for dense ops and for decode attention (its decode rows);
  // prefill attention: the union of its requests' rows, stored as intervals
  std::vector<std::pair<int32_t, int32_t>> rows;
  // decode attention: decode requests [r0, r1); prefill attention: list of prefill requests
  int32_t r0 = 0, r1 = 0;
  std::vector<int32_t> prefill_reqs;
  bool empty = false;
};

struct PlanGraph {
  int32_t n_nano = 1, n_streams = 1;
  int32_t n_dec = 0;  // decode tokens (= decode requests), rows [0, n_dec) of the batch
  std::vector<int32_t> bounds;
  std::vector<NanoOp> ops;                 // in the plan's listed order
  std::vector<std::vector<int32_t>> deps;  // deps[j] = ops j depends on (range intersection)
  std::vector<int32_t> order;              // global issue order (topological)
};

// Build nano-ops, dependencies and a global order from a plan (NULL plan = one nano-batch,
// one stream, kinds in layer order). Checks bounds, the op list and acyclicity.
nf_status build_plan_graph(const BatchLayout& L, const nf_plan* plan, PlanGraph& g, std::string& err);

// The nano-operations of n_layers consecutive layers over one batch, each layer with the
// same plan. Stack op l * n_ops + i is op i of the plan in layer l. Besides every layer's own
// dependencies, the first dense op of layer l + 1 (KQV: it reads the layer input rows)
// depends on the UGD ops of layer l whose rows intersect its rows. `listing` is the order
// the ops are taken in, streams included: layer by layer in the plan's listed order, or,
// when pipelined, with each KQV of layer l + 1 moved up to just after the last layer-l op
// it depends on, so that a stream can start the next layer's nano-batch j while nano-batch
// j + 1 of this layer is still running elsewhere (cross-layer nano-batch pipelining). A
// stream runs its ops in listing order; `order` is a global issue order consistent with
// both that and the dependencies.
struct StackGraph {
  int32_t n_layers = 1, n_ops = 0;        // layers; ops per layer
  std::vector<std::vector<int32_t>> deps;  // per stack op
  std::vector<int32_t> listing, order;
};
nf_status build_stack_graph(const PlanGraph& g, int32_t n_layers, bool pipelined, StackGraph& s, std::string& err);

// One (block, token run) of a KV move between a pool and token-major staging rows: slots
// blk * 16 + [tok0, tok1) <-> staging rows row .. row + tok1 - tok0 - 1.
struct KvMoveItem {
  int32_t blk, tok0, tok1, row;
};
// Validate ranges against a pool of num_blocks blocks and list their moves; check_alias:
// reject two tokens on one slot (NF_E_SLOT_ALIAS). n_rows: total tokens.
nf_status build_kv_moves(const nf_layer_cfg& cfg, const nf_kv_ranges& r, int32_t num_blocks, bool check_alias,
                         std::vector<KvMoveItem>& items, int64_t& n_rows, std::string& err);

// Parent-operation dependency of the layer (does kind b consume a product of kind a?).
bool parent_depends(int32_t a, int32_t b);

// Attention work lists of every nano-batch (host side) and, after upload, device pointers.
struct Meta {
  std::vector<DecodeItem> dec;
  std::vector<CombineItem> comb, pcomb;  // combines of split decode / prefill work
  std::vector<PrefillItem> pf;
  std::vector<int32_t> dec_begin, comb_begin, pf_begin, pcomb_begin;  // size n_nano + 1
  int32_t n_parts = 0;
  const int32_t* d_pos = nullptr;
  const int32_t* d_slot = nullptr;
  const float* d_inv_freq = nullptr;
  const DecodeItem* d_dec = nullptr;
  const CombineItem* d_comb = nullptr;
  const CombineItem* d_pcomb = nullptr;
  const PrefillItem* d_pf = nullptr;
  const int32_t* d_bt = nullptr;
  // dense ops: byte offset of each GEMM's split-K workspace (2 per op: first, second GEMM)
  std::vector<size_t> gemm_ws_off;
};

// Decode split-KV chunks of at most `split` blocks (0 = chosen per nano-op so that its
// (chunk, KV head) units fill the GPU several times; multi-chunk requests get partial slots
// and a combine entry) and prefill tiles with their key chunks (build_prefill_work, chunk
// size pf_chunk keys, 0 = prefill_chunk_keys per nano-op), per nano-batch. Partial slots of all of them are
// distinct (ops of one layer may run concurrently).
void build_work(const BatchLayout& L, const PlanGraph& g, int split, int pf_chunk, int n_q, int n_kv, Meta& M);

}  // namespace nf
