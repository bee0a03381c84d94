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

// One prefill attention work item: 16 consecutive queries of one prefill request.
struct PrefillItem {
  int32_t req;        // request index (row of the block table)
  int32_t token0;     // dense-batch row of the first query of the request
  int32_t q_begin;    // first query (within the request) of this 16-query tile
  int32_t q_len;      // queries of the request
  int32_t prefix;     // cached prefix length
  int32_t pad[3];
};

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
  std::vector<CombineItem> comb;
  std::vector<PrefillItem> pf;
  std::vector<int32_t> dec_begin, comb_begin, pf_begin;  // size n_nano + 1
  int32_t n_parts = 0;
  const int32_t* d_pos = nullptr;
  const int32_t* d_slot = nullptr;
  const float* d_inv_freq = nullptr;
  const DecodeItem* d_dec = nullptr;
  const CombineItem* d_comb = nullptr;
  const PrefillItem* d_pf = nullptr;
  const int32_t* d_bt = nullptr;
  // dense ops: byte offset of each GEMM's split-K workspace (2 per op: first, second GEMM)
  std::vector<size_t> gemm_ws_off;
};

// Decode split-KV chunks of at most `split` blocks (0 = chosen per nano-op so that its
// (chunk, KV head) units fill the GPU several times; multi-chunk requests get partial slots
// and a combine entry) and 16-query prefill tiles (longest first), per nano-batch.
void build_work(const BatchLayout& L, const PlanGraph& g, int split, int n_kv, Meta& M);

}  // namespace nf
