// extern "C" entry points declared in include/tree_attn.h.
//
// Each call validates everything on the host first (plan.cpp), so an invalid
// call enqueues nothing and leaves its outputs untouched; only then are the
// kernel arguments packed and the kernel launched on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "launch.h"
#include "plan.h"

using namespace ta;

namespace {

// Polls (about 2048 cycles apart) a split waits for the other splits of its
// row block before leaving its rows to the last arrival: about 1 ms.
std::atomic<int32_t> g_wait_polls{1000};

// floor(2^32 / d) + 1 (0 for d = 1): the kernels divide x < 2^17 by d < 2^15
// as the high word of x times this (the product overshoots x / d by less
// than 2^-15 < 1 / d, so its integer part is the quotient).
// Verification workspace: the rows' arrival count, then one slot per
// logits row (key and arrival count), kVerifySlot bytes each.
constexpr size_t kVerifyWsBytes = kVerifySlot * (1 + kMaxVerifyRows);

uint32_t div_rcp(int32_t d) {
  return d <= 1 ? 0u : static_cast<uint32_t>((uint64_t{1} << 32) / static_cast<uint64_t>(d) + 1);
}

ta_status device_error(hipError_t e, const char* what) {
  return fail(TA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

int32_t ta_abi_version(void) { return TA_ABI_VERSION; }

void ta_set_split_wait_limit(int32_t polls) { g_wait_polls.store(polls < 0 ? 0 : polls); }

const char* ta_last_error(void) { return last_error(); }

const char* ta_status_string(ta_status s) {
  switch (s) {
    case TA_OK: return "ok";
    case TA_ERR_ARG: return "invalid argument";
    case TA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TA_ERR_CAPACITY: return "cache capacity exceeded";
    case TA_ERR_TREE: return "malformed tree, path or survivor list";
    case TA_ERR_DEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

static_assert(kMaxTree == TA_MAX_TREE, "tree size of the kernels and of the ABI");

ta_status ta_tree_ancestor_bitset(const int32_t* parent, int32_t n_tree, uint64_t* words_out) {
  clear_error();
  if (n_tree > 0 && words_out == nullptr) return fail(TA_ERR_ARG, "words_out is null");
  uint64_t lo[TA_MAX_TREE], hi[TA_MAX_TREE];
  const ta_status st = ancestor_bits(parent, n_tree, lo, hi);
  if (st != TA_OK) return st;
  for (int32_t i = 0; i < n_tree; ++i) {
    words_out[2 * i] = lo[i];
    words_out[2 * i + 1] = hi[i];
  }
  return TA_OK;
}

ta_status ta_tree_ancestor_bits(const int32_t* parent, int32_t n_tree, uint64_t* bits_out) {
  clear_error();
  if (n_tree > 64) return fail(TA_ERR_UNSUPPORTED, "one word per node holds at most 64 nodes");
  return ancestor_bits(parent, n_tree, bits_out, nullptr);
}

ta_status ta_kv_reroot_plan(int32_t prefix_len, int32_t capacity, const int32_t* parent,
                            int32_t n_tree, const int32_t* accepted_path, int32_t n_accepted,
                            const int32_t* surviving_nodes, int32_t n_surviving,
                            int32_t* src_rows_out, int32_t* new_parent, int32_t* new_prefix_len) {
  clear_error();
  return plan_kv_reroot(prefix_len, capacity, parent, n_tree, accepted_path, n_accepted,
                        surviving_nodes, n_surviving, src_rows_out, new_parent, new_prefix_len);
}

size_t ta_tree_attn_rows_workspace_bytes(const ta_kv_cache* cache, int32_t n_q_heads,
                                         int32_t prefix_len, int32_t n_tree, int32_t q_first) {
  clear_error();
  AttnPlan p;
  if (plan_tree_attn(cache, n_q_heads, prefix_len, n_tree, q_first, &p) != TA_OK) return 0;
  return p.ws_bytes;
}

size_t ta_tree_attn_workspace_bytes(const ta_kv_cache* cache, int32_t n_q_heads,
                                    int32_t prefix_len, int32_t n_tree) {
  return ta_tree_attn_rows_workspace_bytes(cache, n_q_heads, prefix_len, n_tree, 0);
}

int32_t ta_tree_attn_rows_num_splits(const ta_kv_cache* cache, int32_t n_q_heads, int32_t prefix_len,
                                     int32_t n_tree, int32_t q_first) {
  clear_error();
  AttnPlan p;
  if (plan_tree_attn(cache, n_q_heads, prefix_len, n_tree, q_first, &p) != TA_OK) return 0;
  return p.splits > 0 ? p.splits : 1;
}

int32_t ta_tree_attn_rows_block_rows(const ta_kv_cache* cache, int32_t n_q_heads, int32_t prefix_len,
                                     int32_t n_tree, int32_t q_first) {
  clear_error();
  AttnPlan p;
  if (plan_tree_attn(cache, n_q_heads, prefix_len, n_tree, q_first, &p) != TA_OK) return 0;
  return p.block_rows;
}

int32_t ta_tree_attn_num_splits(const ta_kv_cache* cache, int32_t n_q_heads, int32_t prefix_len,
                                int32_t n_tree) {
  return ta_tree_attn_rows_num_splits(cache, n_q_heads, prefix_len, n_tree, 0);
}

ta_status ta_tree_attn(const void* q, const ta_kv_cache* cache, int32_t layer,
                       int32_t prefix_len, const int32_t* parent, int32_t n_tree,
                       int32_t n_q_heads, void* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return ta_tree_attn_rows(q, cache, layer, prefix_len, parent, n_tree, 0, n_q_heads, out, workspace,
                           workspace_bytes, stream);
}

ta_status ta_tree_attn_rows(const void* q, const ta_kv_cache* cache, int32_t layer,
                            int32_t prefix_len, const int32_t* parent, int32_t n_tree, int32_t q_first,
                            int32_t n_q_heads, void* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  clear_error();
  return tree_attn_rows_impl(q, cache, layer, prefix_len, parent, n_tree, q_first, n_q_heads, out, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"

namespace ta {

ta_status tree_attn_rows_impl(const void* q, const ta_kv_cache* cache, int32_t layer, int32_t prefix_len,
                              const int32_t* parent, int32_t n_tree, int32_t q_first, int32_t n_q_heads,
                              void* out, void* workspace, size_t workspace_bytes, void* stream) {
  ta_status st = check_cache(cache, true);
  if (st != TA_OK) return st;
  AttnPlan plan;
  st = plan_tree_attn(cache, n_q_heads, prefix_len, n_tree, q_first, &plan);
  if (st != TA_OK) return st;
  if (layer < 0 || layer >= cache->n_layers) return fail(TA_ERR_ARG, "layer out of range");
  TreeAttnArgs a;
  std::memset(&a, 0, sizeof(a));
  st = ancestor_bits(parent, n_tree, a.anc, a.anc_hi);
  if (st != TA_OK) return st;
  if (plan.rows_per_head == 0) return TA_OK;  // no query rows
  if (q == nullptr || out == nullptr) return fail(TA_ERR_ARG, "q or out is null");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(TA_ERR_ARG, "q and out must be 16-byte aligned");
  if (plan.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.ws_bytes)
      return fail(TA_ERR_ARG, "workspace too small: need " + std::to_string(plan.ws_bytes) +
                                  " bytes, got " + std::to_string(workspace_bytes));
    if (reinterpret_cast<uintptr_t>(workspace) & 255)
      return fail(TA_ERR_ARG, "workspace must be 256-byte aligned");
  }
  const size_t es = dtype_bytes(cache->dtype);
  const int64_t head_stride = static_cast<int64_t>(cache->capacity) * cache->head_dim;
  const size_t layer_bytes = static_cast<size_t>(cache->n_kv_heads) * head_stride * es;
  char* ws = static_cast<char*>(workspace);
  a.q = q;
  a.k = static_cast<const char*>(cache->k) + layer * layer_bytes;
  a.v = static_cast<const char*>(cache->v) + layer * layer_bytes;
  a.out = out;
  a.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_o_offset) : nullptr;
  a.ws_ml = plan.ws_bytes ? reinterpret_cast<float2*>(ws + plan.ws_ml_offset) : nullptr;
  a.ws_cnt = plan.ws_bytes ? reinterpret_cast<int32_t*>(ws + plan.ws_cnt_offset) : nullptr;
  a.kv_head_stride = head_stride;
  a.n_q_heads = n_q_heads;
  a.group = plan.group;
  a.n_tree = n_tree;
  a.q_first = q_first;
  a.prefix_len = prefix_len;
  a.total_keys = plan.total_keys;
  a.rows_per_head = plan.rows_per_head;
  a.block_rows = plan.block_rows;
  a.row_blocks = plan.row_blocks;
  a.splits = plan.splits;
  a.n_tiles = plan.n_tiles;
  a.n_units = plan.n_units;
  a.wait_polls = g_wait_polls.load();
  a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(cache->head_dim)));
  a.splits_rcp = div_rcp(plan.splits);
  a.row_blocks_rcp = div_rcp(plan.row_blocks);
  a.group_rcp = div_rcp(plan.group);
  a.split_stages = plan.n_tiles / plan.splits;
  a.split_extra = plan.n_tiles % plan.splits;
  hipError_t e = launch_tree_attn(a, cache->dtype, cache->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "tree_attn launch");
  return TA_OK;
}

}  // namespace ta

extern "C" {

size_t ta_tree_verify_workspace_bytes(int32_t n_tree) {
  clear_error();
  if (n_tree < 0 || n_tree > TA_MAX_TREE) {
    fail(TA_ERR_UNSUPPORTED, "n_tree must be in [0, " + std::to_string(TA_MAX_TREE) + "]");
    return 0;
  }
  return kVerifyWsBytes;
}

ta_status ta_tree_verify(const void* logits, int32_t dtype, int64_t vocab, int64_t row_stride,
                         const int32_t* tokens, const int32_t* parent, int32_t n_tree,
                         int32_t* choice_out, int32_t* result_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  clear_error();
  VerifyArgs a;
  std::memset(&a, 0, sizeof(a));
  ta_status st = ancestor_bits(parent, n_tree, a.anc, a.anc_hi);
  if (st != TA_OK) return st;
  const size_t es = dtype_bytes(dtype);
  if (es == 0) return fail(TA_ERR_UNSUPPORTED, "dtype must be TA_F32 or TA_BF16");
  if (vocab < 1 || vocab > INT32_MAX) return fail(TA_ERR_ARG, "vocab must be in [1, 2^31)");
  if (row_stride < vocab) return fail(TA_ERR_ARG, "row_stride is smaller than vocab");
  if ((static_cast<uint64_t>(row_stride) * es) % 16 != 0)
    return fail(TA_ERR_ARG, "row_stride * element size must be a multiple of 16 bytes");
  if (logits == nullptr || choice_out == nullptr || result_out == nullptr || (n_tree > 0 && tokens == nullptr))
    return fail(TA_ERR_ARG, "logits, tokens, choice_out or result_out is null");
  if (reinterpret_cast<uintptr_t>(logits) & 15) return fail(TA_ERR_ARG, "logits must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(tokens) | reinterpret_cast<uintptr_t>(choice_out) |
       reinterpret_cast<uintptr_t>(result_out)) & 3)
    return fail(TA_ERR_ARG, "tokens, choice_out and result_out must be 4-byte aligned");
  if (workspace == nullptr || workspace_bytes < kVerifyWsBytes)
    return fail(TA_ERR_ARG, "workspace too small: need " + std::to_string(kVerifyWsBytes) + " bytes, got " +
                                std::to_string(workspace_bytes));
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(TA_ERR_ARG, "workspace must be 256-byte aligned");
  for (int32_t i = 0; i < n_tree; ++i) a.parent[i] = static_cast<int8_t>(parent[i]);
  char* ws = static_cast<char*>(workspace);
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = vocab;
  a.rows = n_tree + 1;
  a.n_tree = n_tree;
  a.tokens = tokens;
  a.choice = choice_out;
  a.result = result_out;
  a.ws = ws;
  hipError_t e = launch_tree_verify(a, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "tree_verify launch");
  return TA_OK;
}

size_t ta_tree_expand_workspace_bytes(int32_t w) {
  clear_error();
  if (w < 1 || w > kExpandMaxRows) {
    fail(TA_ERR_UNSUPPORTED, "w must be in [1, " + std::to_string(kExpandMaxRows) + "]");
    return 0;
  }
  return static_cast<size_t>(kExpandChunkBase) + static_cast<size_t>(w) * kExpandMaxChunks * kExpandChunkSlot;
}

ta_status ta_tree_expand(const void* logits, int32_t dtype, int64_t vocab, int64_t row_stride,
                         const float* path_scores, int32_t w, int32_t k, int32_t* leaf_out,
                         int32_t* token_out, float* score_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  clear_error();
  const size_t es = dtype_bytes(dtype);
  if (es == 0) return fail(TA_ERR_UNSUPPORTED, "dtype must be TA_F32 or TA_BF16");
  if (w < 1 || w > kExpandMaxRows)
    return fail(TA_ERR_UNSUPPORTED, "w must be in [1, " + std::to_string(kExpandMaxRows) + "]");
  if (k < 1 || k > kExpandMaxK) return fail(TA_ERR_UNSUPPORTED, "k must be in [1, " + std::to_string(kExpandMaxK) + "]");
  const int64_t max_vocab = static_cast<int64_t>(kExpandMaxChunks) * kExpandChunk;
  if (vocab < 1 || vocab > max_vocab)
    return fail(TA_ERR_UNSUPPORTED, "vocab must be in [1, " + std::to_string(max_vocab) + "]");
  if (static_cast<int64_t>(k) > static_cast<int64_t>(w) * vocab) return fail(TA_ERR_ARG, "k exceeds w * vocab");
  if (row_stride < vocab) return fail(TA_ERR_ARG, "row_stride is smaller than vocab");
  if ((static_cast<uint64_t>(row_stride) * es) % 16 != 0)
    return fail(TA_ERR_ARG, "row_stride * element size must be a multiple of 16 bytes");
  if (logits == nullptr || path_scores == nullptr || leaf_out == nullptr || token_out == nullptr ||
      score_out == nullptr)
    return fail(TA_ERR_ARG, "logits, path_scores or an output is null");
  if (reinterpret_cast<uintptr_t>(logits) & 15) return fail(TA_ERR_ARG, "logits must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(path_scores) | reinterpret_cast<uintptr_t>(leaf_out) |
       reinterpret_cast<uintptr_t>(token_out) | reinterpret_cast<uintptr_t>(score_out)) & 3)
    return fail(TA_ERR_ARG, "path_scores and the outputs must be 4-byte aligned");
  const size_t need = ta_tree_expand_workspace_bytes(w);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(TA_ERR_ARG, "workspace too small: need " + std::to_string(need) + " bytes, got " +
                                std::to_string(workspace_bytes));
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(TA_ERR_ARG, "workspace must be 256-byte aligned");
  ExpandArgs a;
  std::memset(&a, 0, sizeof(a));
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = vocab;
  a.path_scores = path_scores;
  a.w = w;
  a.k = k;
  a.chunks = static_cast<int32_t>((vocab + kExpandChunk - 1) / kExpandChunk);
  a.ws_bytes = static_cast<int32_t>(need);
  a.leaf_out = leaf_out;
  a.token_out = token_out;
  a.score_out = score_out;
  a.ws = static_cast<char*>(workspace);
  hipError_t e = launch_tree_expand(a, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "tree_expand launch");
  return TA_OK;
}

ta_status ta_kv_reroot(const ta_kv_cache* cache, int32_t prefix_len, const int32_t* parent,
                       int32_t n_tree, const int32_t* accepted_path, int32_t n_accepted,
                       const int32_t* surviving_nodes, int32_t n_surviving, int32_t* new_parent,
                       int32_t* new_prefix_len, void* stream) {
  clear_error();
  ta_status st = check_cache(cache, true);
  if (st != TA_OK) return st;
  RerootArgs a;
  std::memset(&a, 0, sizeof(a));
  int32_t np_tmp[TA_MAX_TREE];
  int32_t npl_tmp = 0;
  st = plan_kv_reroot(prefix_len, cache->capacity, parent, n_tree, accepted_path, n_accepted,
                      surviving_nodes, n_surviving, a.src, np_tmp, &npl_tmp);
  if (st != TA_OK) return st;
  if (new_prefix_len == nullptr || (n_surviving > 0 && new_parent == nullptr))
    return fail(TA_ERR_ARG, "output pointer is null");
  const int32_t rows = n_accepted + n_surviving;
  bool moves = false;
  for (int32_t k = 0; k < rows; ++k) moves |= a.src[k] != prefix_len + k;
  if (moves) {
    const size_t es = dtype_bytes(cache->dtype);
    a.k = static_cast<char*>(cache->k);
    a.v = static_cast<char*>(cache->v);
    a.row_bytes = static_cast<int32_t>(cache->head_dim * es);
    a.plane_bytes = static_cast<int64_t>(cache->capacity) * a.row_bytes;
    a.n_planes = cache->n_layers * cache->n_kv_heads;
    a.n_rows = rows;
    a.dst0 = prefix_len;
    // Every column of a plane in one workgroup while a thread's share stays
    // within kRerootItemsPerThread: its loads are then all in flight at once,
    // and a launch of many planes needs only one workgroup per plane.
    const int32_t cols = a.row_bytes / 16;
    int32_t gcols = cols;
    while (gcols > 1 && rows * gcols > kRerootItemsPerThread * kRerootThreads) gcols /= 2;
    a.col_groups = cols / gcols;
    a.gcols_rcp = div_rcp(gcols);
    hipError_t e = launch_kv_reroot(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_error(e, "kv_reroot launch");
  }
  for (int32_t k = 0; k < n_surviving; ++k) new_parent[k] = np_tmp[k];
  *new_prefix_len = npl_tmp;
  return TA_OK;
}

}  // extern "C"
