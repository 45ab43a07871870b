// Host-side validation and planning (no HIP). See plan.h.
//
// The semantics follow the SwiftSpec pages (arXiv 2506.11309, Pith review
// page): "What carries the argument" fixes the [verified prefix | tree] cache
// layout and the re-root at the last verified token; "Core claim" says the
// verified tokens join the prefix and the surviving tree states are packed
// right after it.
#include "plan.h"

#include <algorithm>
#include <string>

namespace ta {

namespace {
thread_local std::string g_last_error;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace

ta_status fail(ta_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
void clear_error() { g_last_error.clear(); }
const char* last_error() { return g_last_error.c_str(); }

size_t dtype_bytes(int32_t dtype) {
  return dtype == TA_F32 ? 4 : dtype == TA_BF16 ? 2 : 0;
}

ta_status check_parent(const int32_t* parent, int32_t n) {
  if (n < 0) return fail(TA_ERR_ARG, "n_tree is negative");
  if (n > TA_MAX_TREE)
    return fail(TA_ERR_UNSUPPORTED, "n_tree " + std::to_string(n) + " exceeds " +
                                        std::to_string(TA_MAX_TREE));
  if (n > 0 && parent == nullptr) return fail(TA_ERR_ARG, "parent is null");
  for (int32_t i = 0; i < n; ++i) {
    if (!(parent[i] == -1 || (parent[i] >= 0 && parent[i] < i)))
      return fail(TA_ERR_TREE, "parent[" + std::to_string(i) + "] = " +
                                   std::to_string(parent[i]) + " is neither -1 nor in [0, " +
                                   std::to_string(i) + ")");
  }
  return TA_OK;
}

ta_status ancestor_bits(const int32_t* parent, int32_t n, uint64_t* lo, uint64_t* hi) {
  ta_status st = check_parent(parent, n);
  if (st != TA_OK) return st;
  if (n > 0 && lo == nullptr) return fail(TA_ERR_ARG, "bits_out is null");
  if (n > 64 && hi == nullptr) return fail(TA_ERR_UNSUPPORTED, "more than 64 nodes need two words per node");
  // parent[i] < i, so the sets of parent[i] are final when node i is reached.
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = parent[i];
    lo[i] = (i < 64 ? uint64_t{1} << i : 0) | (p < 0 ? 0 : lo[p]);
    if (hi != nullptr) hi[i] = (i >= 64 ? uint64_t{1} << (i - 64) : 0) | (p < 0 ? 0 : hi[p]);
  }
  return TA_OK;
}

ta_status check_cache(const ta_kv_cache* c, bool need_ptrs) {
  if (c == nullptr) return fail(TA_ERR_ARG, "cache descriptor is null");
  if (c->dtype != TA_F32 && c->dtype != TA_BF16)
    return fail(TA_ERR_UNSUPPORTED, "cache dtype must be TA_F32 or TA_BF16");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(TA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->n_layers < 1 || c->n_kv_heads < 1 || c->capacity < 1)
    return fail(TA_ERR_ARG, "n_layers, n_kv_heads and capacity must be positive");
  if (need_ptrs) {
    if (c->k == nullptr || c->v == nullptr) return fail(TA_ERR_ARG, "cache k or v is null");
    if ((reinterpret_cast<uintptr_t>(c->k) | reinterpret_cast<uintptr_t>(c->v)) & 15)
      return fail(TA_ERR_ARG, "cache k and v must be 16-byte aligned");
  }
  return TA_OK;
}

ta_status plan_tree_attn(const ta_kv_cache* cache, int32_t n_q_heads, int32_t prefix_len,
                         int32_t n_tree, int32_t q_first, AttnPlan* plan) {
  ta_status st = check_cache(cache, false);
  if (st != TA_OK) return st;
  if (n_tree < 0 || n_tree > TA_MAX_TREE)
    return fail(n_tree < 0 ? TA_ERR_ARG : TA_ERR_UNSUPPORTED,
                "n_tree must be in [0, " + std::to_string(TA_MAX_TREE) + "]");
  if (prefix_len < 0) return fail(TA_ERR_ARG, "prefix_len is negative");
  if (q_first < 0 || q_first > n_tree) return fail(TA_ERR_ARG, "q_first must be in [0, n_tree]");
  if (n_q_heads < 1 || n_q_heads % cache->n_kv_heads != 0)
    return fail(TA_ERR_UNSUPPORTED, "n_q_heads must be a positive multiple of n_kv_heads");
  const int32_t group = n_q_heads / cache->n_kv_heads;
  if (group > 16) return fail(TA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  if (static_cast<int64_t>(prefix_len) + n_tree > cache->capacity)
    return fail(TA_ERR_CAPACITY, "prefix_len + n_tree = " +
                                     std::to_string(static_cast<int64_t>(prefix_len) + n_tree) +
                                     " exceeds capacity " + std::to_string(cache->capacity));
  // The kernels address one KV head's [prefix | tree] rows, and the query
  // rows of one call, through raw-buffer descriptors whose byte ranges and
  // per-lane offsets are 32-bit (loads run up to four 64-key stages past a
  // range's end, where the range check returns zeros); refuse shapes whose
  // ranges could wrap instead of mis-addressing them.
  const int64_t es = static_cast<int64_t>(dtype_bytes(cache->dtype));
  const int64_t kMaxRange = INT32_MAX - (int64_t{1} << 20);
  if ((static_cast<int64_t>(prefix_len) + n_tree) * cache->head_dim * es > kMaxRange)
    return fail(TA_ERR_UNSUPPORTED, "prefix_len + n_tree = " +
                                        std::to_string(static_cast<int64_t>(prefix_len) + n_tree) +
                                        " keys of one KV head exceed the kernels' 32-bit byte range");
  if (static_cast<int64_t>(n_tree - q_first) * n_q_heads * cache->head_dim * es > kMaxRange)
    return fail(TA_ERR_UNSUPPORTED, "the query rows of one call exceed the kernels' 32-bit byte range");
  AttnPlan p;
  p.head_dim = cache->head_dim;
  p.group = group;
  p.rows_per_head = group * (n_tree - q_first);
  // bf16 heads of at most 64 rows run the sparse-block instance, whose blocks
  // are 64 rows; 128 rows otherwise (64 below when CUs would stay idle)
  const bool small = cache->dtype == TA_BF16 && p.rows_per_head <= kRowsPerBlock / 2;
  p.block_rows = small ? kRowsPerBlock / 2 : kRowsPerBlock;
  p.row_blocks = (p.rows_per_head + kRowsPerBlock - 1) / kRowsPerBlock;
  p.total_keys = prefix_len + n_tree;
  p.n_tiles = (p.total_keys + kKeyTile - 1) / kKeyTile;
  if (p.rows_per_head == 0) {  // no query rows: nothing to do
    *plan = p;
    return TA_OK;
  }
  const int32_t base_units = cache->n_kv_heads * p.row_blocks;
  // Aim for every CU busy with all splits resident at once (the split merge
  // waits for its partners): the bf16 kernel runs one workgroup per CU, the
  // fp32 one two (one for head_dim 128).
  const bool one_per_cu = cache->dtype == TA_BF16 || cache->head_dim == 128;
  const int32_t target = one_per_cu ? kTargetUnits / 2 : kTargetUnits;
  const int32_t cap = std::max(1, p.n_tiles / kMinTilesPerSplit);
  auto splits_for = [&](int32_t base) {
    const int32_t want = (target + base - 1) / base;
    return std::max(1, std::min(std::min(want, cap), kMaxSplits));
  };
  p.splits = splits_for(base_units);
  p.n_units = base_units * p.splits;
  // bf16: 64-row blocks (each block's two real row tiles run one wave per
  // SIMD, the other four waves only load) where they give more units than
  // 128-row blocks without passing the target, or as many units with
  // splits of at most kMaxStagesHalfBlocks stages: there half the partial
  // rows and longer splits outweigh the slower loop of a one-wave SIMD.
  if (cache->dtype == TA_BF16 && p.rows_per_head > kRowsPerBlock / 2 && p.n_units <= target) {
    const int32_t half = kRowsPerBlock / 2;
    const int32_t blocks = (p.rows_per_head + half - 1) / half;
    const int32_t splits = splits_for(cache->n_kv_heads * blocks);
    const int64_t units = static_cast<int64_t>(cache->n_kv_heads) * blocks * splits;
    const bool short_splits = (p.n_tiles + splits - 1) / splits <= kMaxStagesHalfBlocks;
    if ((units > p.n_units || (units == p.n_units && short_splits)) && units <= target) {
      p.block_rows = half;
      p.row_blocks = blocks;
      p.splits = splits;
      p.n_units = static_cast<int32_t>(units);
    }
  }
  const int32_t base_groups = cache->n_kv_heads * p.row_blocks;
  // The kernels split a workgroup id into (group, split) and a group into
  // (KV head, row block) with a multiply-high division that is exact for
  // dividends below 2^17.
  if (p.n_units >= kMaxUnits)
    return fail(TA_ERR_UNSUPPORTED, std::to_string(p.n_units) + " work units (KV heads x row blocks x splits) "
                                    "exceed " + std::to_string(kMaxUnits - 1));
  if (p.splits > 1) {
    if (base_groups > kMaxGroups)
      return fail(TA_ERR_UNSUPPORTED, "more than " + std::to_string(kMaxGroups) +
                                          " (KV head, row block) groups need a split");
    const size_t units = static_cast<size_t>(p.n_units);
    p.ws_cnt_offset = 0;
    p.ws_ml_offset = kCounterBytes;
    const size_t ml_bytes = units * kRowsPerBlock * 2 * sizeof(float);
    p.ws_o_offset = align_up(p.ws_ml_offset + ml_bytes, 256);
    // partial rows in fp32 for every cache dtype
    const size_t o_bytes = units * kRowsPerBlock * p.head_dim * sizeof(float);
    p.ws_bytes = align_up(p.ws_o_offset + o_bytes, 256);
  }
  *plan = p;
  return TA_OK;
}

ta_status plan_kv_reroot(int32_t prefix_len, int32_t capacity, const int32_t* parent,
                         int32_t n_tree, const int32_t* path, int32_t n_path,
                         const int32_t* surv, int32_t n_surv, int32_t* src_rows,
                         int32_t* new_parent, int32_t* new_prefix_len) {
  ta_status st = check_parent(parent, n_tree);
  if (st != TA_OK) return st;
  if (prefix_len < 0 || capacity < 0) return fail(TA_ERR_ARG, "prefix_len/capacity negative");
  if (static_cast<int64_t>(prefix_len) + n_tree > capacity)
    return fail(TA_ERR_CAPACITY, "prefix_len + n_tree exceeds capacity");
  if (n_path < 0 || n_surv < 0) return fail(TA_ERR_ARG, "negative path or survivor count");
  if ((n_path > 0 && path == nullptr) || (n_surv > 0 && surv == nullptr))
    return fail(TA_ERR_ARG, "path or survivor list is null");
  if (n_path + n_surv > n_tree) return fail(TA_ERR_TREE, "more path+survivor nodes than tree nodes");
  if (new_prefix_len == nullptr || (n_surv > 0 && new_parent == nullptr))
    return fail(TA_ERR_ARG, "output pointer is null");

  // 0 = unused, 1 = on the path, 2 = survivor (with new index in `pos`).
  int8_t role[TA_MAX_TREE] = {0};
  int32_t pos[TA_MAX_TREE];
  for (int32_t k = 0; k < n_path; ++k) {
    const int32_t a = path[k];
    if (a < 0 || a >= n_tree) return fail(TA_ERR_TREE, "accepted node out of range");
    const int32_t want = k == 0 ? -1 : path[k - 1];
    if (parent[a] != want)
      return fail(TA_ERR_TREE, "accepted path is not a chain from a first-level node (position " +
                                   std::to_string(k) + ")");
    role[a] = 1;
  }
  const int32_t last = n_path > 0 ? path[n_path - 1] : -1;
  for (int32_t k = 0; k < n_surv; ++k) {
    const int32_t s = surv[k];
    if (s < 0 || s >= n_tree) return fail(TA_ERR_TREE, "survivor out of range");
    if (k > 0 && s <= surv[k - 1]) return fail(TA_ERR_TREE, "survivors must be strictly ascending");
    if (role[s] == 1) return fail(TA_ERR_TREE, "survivor " + std::to_string(s) + " is on the path");
    // Ascending order means the parent, if it is a survivor, was already seen.
    const int32_t p = parent[s];
    if (!(p == last || (p >= 0 && role[p] == 2)))
      return fail(TA_ERR_TREE, "survivor " + std::to_string(s) + " does not hang below the last "
                               "accepted node");
    role[s] = 2;
    pos[s] = k;
  }
  // Everything is valid: write the outputs.
  if (src_rows != nullptr) {
    for (int32_t k = 0; k < n_path; ++k) src_rows[k] = prefix_len + path[k];
    for (int32_t k = 0; k < n_surv; ++k) src_rows[n_path + k] = prefix_len + surv[k];
  }
  for (int32_t k = 0; k < n_surv; ++k) {
    const int32_t p = parent[surv[k]];
    new_parent[k] = p == last ? -1 : pos[p];
  }
  *new_prefix_len = prefix_len + n_path;
  return TA_OK;
}

}  // namespace ta
