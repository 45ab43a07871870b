// Kernel argument blocks and launchers shared by the C ABI (api.cpp) and the
// HIP kernels. Everything here is passed to the device by value.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tree_attn.h"

namespace ta {

// Tree nodes per call (the C ABI's TA_MAX_TREE): two 64-bit ancestor words.
constexpr int kMaxTree = 128;

struct TreeAttnArgs {
  const void* q;            // [n_tree][n_q_heads][D]
  const void* k;            // layer base: [n_kv_heads][capacity][D]
  const void* v;
  void* out;                // like q
  float* ws_o;              // split partials, see AttnPlan
  float2* ws_ml;
  int32_t* ws_cnt;          // kGroupWords words per (KV head, row block) group
  int64_t kv_head_stride;   // elements from one KV head to the next (capacity * D)
  int32_t n_q_heads;
  int32_t group;            // query heads per KV head
  int32_t n_tree;           // tree nodes (all of them are keys)
  int32_t q_first;          // the query rows are tree nodes q_first .. n_tree-1
  int32_t prefix_len;
  int32_t total_keys;       // prefix_len + n_tree
  int32_t rows_per_head;    // group * (n_tree - q_first)
  int32_t block_rows;       // query rows per row block: 128, or 64 (bf16, see the plan)
  int32_t row_blocks;
  int32_t splits;
  int32_t n_tiles;
  int32_t n_units;
  int32_t wait_polls;       // bound of the wait for the other splits of a group
  float scale_log2;         // log2(e) / sqrt(D)
  // Reciprocals for the kernels' small divisions: floor(2^32 / d) + 1 for a
  // divisor d > 1, 0 for d = 1 (see div_small in the kernel source).
  uint32_t splits_rcp;
  uint32_t row_blocks_rcp;
  uint32_t group_rcp;
  // Split s covers stages [s * split_stages + min(s, split_extra), ...) and
  // one stage more than split_stages when s < split_extra.
  int32_t split_stages;     // n_tiles / splits
  int32_t split_extra;      // n_tiles % splits
  // Ancestor-or-self set of each tree node: anc[i] holds nodes 0..63,
  // anc_hi[i] nodes 64..127 (zero for trees of up to 64 nodes).
  uint64_t anc[kMaxTree];
  uint64_t anc_hi[kMaxTree];
};

hipError_t launch_tree_attn(const TreeAttnArgs& a, int32_t dtype, int32_t head_dim,
                            hipStream_t stream);

// ta_tree_attn_rows without the error reset: validation, planning and the
// launch, on a caller-owned workspace (api.cpp) or the library's static
// scratch (noalloc.hip).
ta_status tree_attn_rows_impl(const void* q, const ta_kv_cache* cache, int32_t layer, int32_t prefix_len,
                              const int32_t* parent, int32_t n_tree, int32_t q_first, int32_t n_q_heads,
                              void* out, void* workspace, size_t workspace_bytes, void* stream);

struct RerootArgs {
  char* k;                  // cache base (all layers)
  char* v;
  int64_t plane_bytes;      // capacity * row_bytes: one (layer, KV head) plane
  int32_t row_bytes;        // head_dim * element size
  int32_t n_planes;         // n_layers * n_kv_heads
  int32_t n_rows;           // rows to place: n_accepted + n_surviving
  int32_t dst0;             // first destination slot (= prefix_len)
  int32_t col_groups;       // column groups per plane (grid.y)
  uint32_t gcols_rcp;       // 2^32 / (columns per group) + 1, 0 for one column: item -> (row, column)
  int32_t src[kMaxTree];    // source slot of destination slot dst0 + k
};

// Workgroup size and (row, 16-byte column) items per thread of the re-root kernel.
constexpr int kRerootThreads = 256;
constexpr int kRerootItemsPerThread = 8;

hipError_t launch_kv_reroot(const RerootArgs& a, hipStream_t stream);

// Rows of one verification: the virtual root and up to kMaxTree nodes.
constexpr int kMaxVerifyRows = kMaxTree + 1;
// Bytes per row slot of the verification workspace (one slot per cache line
// pair, so that the rows' atomics do not share lines).
constexpr int kVerifySlot = 64;

struct VerifyArgs {
  const void* logits;       // rows of the target's logits, row_stride elements apart
  int64_t row_stride;       // elements; row_stride * element size is a multiple of 16
  int64_t vocab;            // values per row, < 2^31
  int32_t rows;             // n_tree + 1
  int32_t n_tree;
  const int32_t* tokens;    // [n_tree] drafted token per node
  int32_t* choice;          // [rows] arg-max per row
  int32_t* result;          // [n_tree + 2]: m, bonus, accepted path, -1 padding
  char* ws;                 // workspace, zero between calls: the arrival count of
                            // rows at 0, then per row r at kVerifySlot * (1 + r)
                            // its 8-byte key and its 4-byte arrival count
  uint64_t anc[kMaxTree];   // ancestor-or-self set per node: nodes 0..63
  uint64_t anc_hi[kMaxTree];  // nodes 64..127
  int8_t parent[kMaxTree];
};

hipError_t launch_tree_verify(const VerifyArgs& a, int32_t dtype, hipStream_t stream);

// Maximum-likelihood expansion: up to 64 frontier leaves, k <= 16 new nodes,
// vocabularies of up to 64 chunks of 4096 logits.
constexpr int kExpandChunk = 4096;       // logits per workgroup
constexpr int kExpandMaxK = 16;
constexpr int kExpandMaxRows = 64;
constexpr int kExpandMaxChunks = 64;
// Workspace layout (zero between calls except where written before read):
// the leaves' arrival count at 0; leaf r's arrival count at
// kExpandRowCount * (1 + r); leaf r's k (score, token) at kExpandRowBase +
// r * kExpandRowSlot; chunk c of leaf r's (max, sum) and k keys at
// kExpandChunkBase + (r * kExpandMaxChunks + c) * kExpandChunkSlot.
constexpr int kExpandRowCount = 64;
constexpr int kExpandRowBase = 8192;
constexpr int kExpandRowSlot = 8 * kExpandMaxK;
constexpr int kExpandChunkBase = 16384;
constexpr int kExpandChunkSlot = 256;

struct ExpandArgs {
  const void* logits;        // w rows of draft logits, row_stride elements apart
  int64_t row_stride;
  int64_t vocab;
  const float* path_scores;  // [w]
  int32_t w;                 // frontier leaves
  int32_t k;                 // new nodes
  int32_t chunks;            // ceil(vocab / kExpandChunk)
  int32_t ws_bytes;
  int32_t* leaf_out;         // [k]
  int32_t* token_out;        // [k]
  float* score_out;          // [k]
  char* ws;
};

hipError_t launch_tree_expand(const ExpandArgs& a, int32_t dtype, hipStream_t stream);

}  // namespace ta
