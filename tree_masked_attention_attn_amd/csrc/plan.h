// Host-side validation and planning for the tree-attention library.
// Plain C++ (no HIP): it is compiled into the library and also builds on its
// own with g++ for sanitizer runs.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "tree_attn.h"

namespace ta {

// Records `msg` as the calling thread's last error and returns `st`.
ta_status fail(ta_status st, const std::string& msg);
void clear_error();
const char* last_error();

// parent[i] in {-1} U [0, i) for every i < n.
ta_status check_parent(const int32_t* parent, int32_t n);

// Root path of i, self included, as a 128-bit set split in two words:
// lo[i] holds nodes 0..63, hi[i] nodes 64..127 (hi may be null when n <= 64).
ta_status ancestor_bits(const int32_t* parent, int32_t n, uint64_t* lo, uint64_t* hi);

// Validates a KV-cache descriptor (pointers may be null when `need_ptrs` is false).
ta_status check_cache(const ta_kv_cache* c, bool need_ptrs);

// Tiling of one ta_tree_attn call. A "work unit" is one workgroup:
// (KV head g, block of block_rows query rows, prefix split s).
struct AttnPlan {
  int32_t head_dim = 0;
  int32_t group = 0;           // query heads per KV head
  int32_t rows_per_head = 0;   // group * (n_tree - q_first): query rows per KV head
  int32_t block_rows = 0;      // query rows per row block: kRowsPerBlock, or half of it (bf16)
  int32_t row_blocks = 0;      // ceil(rows_per_head / block_rows)
  int32_t total_keys = 0;      // prefix_len + n_tree
  int32_t n_tiles = 0;         // ceil(total_keys / kKeyTile): key stages
  int32_t splits = 0;          // key-range splits per row block
  int32_t n_units = 0;         // n_kv_heads * row_blocks * splits
  // Workspace layout (only when splits > 1). The arrival counters always sit
  // at offset 0 in a fixed-size region, whatever the shape, so a workspace
  // that calls of different shapes share never finds partial data of an
  // earlier call where it expects a counter.
  size_t ws_cnt_offset = 0;    // int32 x4 per group: arrivals, pad, give-up bits, pad
  size_t ws_ml_offset = 0;     // fp32 (max, sum) pairs [units][kRowsPerBlock][2] (block_rows used)
  size_t ws_o_offset = 0;      // partial outputs [units][kRowsPerBlock][head_dim], fp32 (block_rows used)
  size_t ws_bytes = 0;
};

constexpr int32_t kKeyTile = 64;       // keys per LDS stage (two 32-key MFMA sub-tiles)
constexpr int32_t kTilesPerBlock = 4;  // 32-row MFMA tiles per row block (the fp32 kernel: one per wave)
constexpr int32_t kRowsPerTile = 32;   // query rows per MFMA tile (one 32-wide MFMA N tile)
constexpr int32_t kRowsPerBlock = kTilesPerBlock * kRowsPerTile;
constexpr int32_t kTargetUnits = 512;  // 2 workgroups per CU on a 256-CU part (half that for one per CU)
// At least 4 key stages per split: below that, the fixed cost of a unit
// (first loads, hand-off, merge) and the partial rows it writes outweigh the
// extra CUs (Llama-3-8B verify, 33 stages: 8 splits on 128 CUs beat 16 on 256
// by 7 percent; 6, 10 and 12 splits were slower still).
constexpr int32_t kMinTilesPerSplit = 4;
// At most 16 splits per row block (the give-up word would have room for 32):
// past 16, the hand-off and merge of the extra partials cost more than the
// shorter key ranges save, also when that leaves CUs idle (measured on a
// bs=8 verify step and a one-row-block draft expansion: 16 splits beat 32 by
// 10 to 25 percent).
constexpr int32_t kMaxSplits = 16;
// 64-row blocks at the unit count of 128-row ones only while their splits
// stay this short. Measured on MI355X, per-launch events, 64- against
// 128-row blocks at 256 units: 9 stages per split -5 to -6% (head_dim 64
// and 128), 17 stages +0% (128) and +4% (64), 25 to 33 stages +12%.
constexpr int32_t kMaxStagesHalfBlocks = 12;
constexpr int32_t kMaxGroups = 4096;   // (KV head, row block) groups with counters
constexpr int32_t kMaxUnits = 1 << 17; // the kernels' index divisions are exact below this
constexpr int32_t kGroupWords = 4;     // arrival count, unused, give-up bits, unused
constexpr size_t kCounterBytes = kMaxGroups * kGroupWords * sizeof(int32_t);

ta_status plan_tree_attn(const ta_kv_cache* cache, int32_t n_q_heads, int32_t prefix_len,
                         int32_t n_tree, int32_t q_first, AttnPlan* plan);

// Re-root plan: src_rows[k] = prefix_len + order[k], order = path ++ survivors.
ta_status plan_kv_reroot(int32_t prefix_len, int32_t capacity, const int32_t* parent,
                         int32_t n_tree, const int32_t* path, int32_t n_path,
                         const int32_t* surv, int32_t n_surv, int32_t* src_rows,
                         int32_t* new_parent, int32_t* new_prefix_len);

size_t dtype_bytes(int32_t dtype);

}  // namespace ta
