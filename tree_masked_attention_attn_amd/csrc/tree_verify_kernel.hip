// Greedy tree verification for gfx950: per-row arg-max of the target's
// logits and the accepted path of the draft tree, in one launch.
//
// SwiftSpec (arXiv 2506.11309), Pith review page, "What carries the argument"
// and the referee report's summary: the target model checks the draft tree as
// a whole, the verified tokens join the prefix and the tree re-roots at the
// last verified token. As in tree-based verification (SpecInfer, in the same
// page's reference list), the target scores every tree node in one pass; its
// logits row 0 belongs to the virtual root (the last verified token) and row
// 1 + i to tree node i. Under greedy decoding node i is accepted when its
// drafted token is the target's arg-max at its parent and every ancestor was
// accepted; the deepest accepted node (lowest index among equally deep ones)
// ends the accepted path, and the target's arg-max there is the bonus token.
//
// Work split. Reading the logits is the whole cost (HBM-bound: every byte is
// read once), so the grid is (vocab chunk, row): each workgroup streams one
// chunk of one row with 16-byte loads, reduces it to one 64-bit key and
// folds the key into its row's slot with a device-scope atomic max. The key
// orders candidates by value, then by lowest index, so the maximum key is the
// row's first maximum whatever order the workgroups finish in. Arrival is
// counted in two levels of wrapping counts: the chunks of a row count in on
// the row's slot, the last of them counts the row in on one shared count,
// and the last row's last chunk goes on (one count per address takes a
// row's chunks or the rows, never the whole grid: device-scope atomics on
// one address serialise). That workgroup reads and clears every slot (atomic
// exchange with zero), writes the arg-max of each row and finds the accepted
// path with one wave: a ballot of the matching nodes, then each node's
// ancestor bitset tells whether its whole root path matched.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "launch.h"
#include "tree_attn.h"
#include "wave_ops.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float to_float(T x) {
  if constexpr (std::is_same_v<T, float>)
    return x;
  else
    return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) << 16);
}

// Vectors of 16 bytes per thread and chunk (kUnroll loads in flight per
// thread): 16 KB chunks, 16 of a 128256-entry bf16 row, 1040 workgroups for
// 65 rows. Measured faster than 8, 32, 64 or 256 KB chunks and than 512- or
// 1024-thread workgroups: the latency chain after the loads is fixed, so the
// loads should finish as early as possible.
constexpr int kUnroll = 4;

template <typename T>
__global__ __launch_bounds__(kThreads) void tree_verify_kernel(const VerifyArgs a) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y;
  const T* x = static_cast<const T*>(a.logits) + static_cast<size_t>(row) * a.row_stride;
  const int64_t full_vecs = a.vocab / EPV;  // whole vectors; the rest is the tail
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + tid;
  // Inputs of the path search, loaded early by every workgroup (only the
  // last one uses them) so that their latency hides under the logits': the
  // drafted token, ancestor set (two words: nodes 0..63, 64..127) and parent
  // of nodes `lane` (h = 0) and `lane + 64` (h = 1).
  bool live[2];
  int tok[2], par[2];
  u64 anc_lo[2], anc_hi[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    live[h] = wave == 0 && i < a.n_tree;
    tok[h] = live[h] ? a.tokens[i] : 0;
    anc_lo[h] = live[h] ? a.anc[i] : 0ull;
    anc_hi[h] = live[h] ? a.anc_hi[i] : 0ull;
    par[h] = live[h] ? a.parent[i] : 0;
  }

  // Each thread scans its elements in ascending index order and keeps the
  // first maximum; it starts from its first element's index with -inf, which
  // is right also when all of its elements are -inf.
  float best = -__builtin_huge_valf();
  uint32_t bidx = 0;
  bool any = false;
  u32x4 buf[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int64_t vi = v0 + j * kThreads;
    if (vi < full_vecs) buf[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + vi);
  }
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int64_t vi = v0 + j * kThreads;
    if (vi < full_vecs) {
      if (!any) {
        any = true;
        bidx = static_cast<uint32_t>(vi * EPV);
      }
      const T* e = reinterpret_cast<const T*>(&buf[j]);
#pragma unroll
      for (int t = 0; t < EPV; ++t) {
        const float f = to_float(e[t]);
        if (f > best) {
          best = f;
          bidx = static_cast<uint32_t>(vi * EPV + t);
        }
      }
    }
  }
  // Tail (vocab not a multiple of EPV): the thread that would own vector
  // full_vecs reads the remaining elements one by one.
  for (int j = 0; j < kUnroll; ++j) {
    if (v0 + j * kThreads == full_vecs) {
      for (int64_t i = full_vecs * EPV; i < a.vocab; ++i) {
        const float f = to_float(x[i]);
        if (!any) {
          any = true;
          bidx = static_cast<uint32_t>(i);
        }
        if (f > best) {
          best = f;
          bidx = static_cast<uint32_t>(i);
        }
      }
    }
  }

  __shared__ u64 s_key[kThreads / 64];
  __shared__ int s_last;
  __shared__ int s_choice[kMaxVerifyRows];
  u64 key = wave_max_u64(any ? cand_key(best, bidx) : 0ull);
  if (lane == 0) s_key[wave] = key;
  __syncthreads();
  if (tid == 0) {
    key = s_key[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) key = s_key[w] > key ? s_key[w] : key;
    // Wait for the returning atomic before counting in: the count then
    // announces a max that is already performed at the device coherence
    // point, where the last workgroup's exchange reads it. Each count is
    // taken only once the one before it has returned.
    char* slot = a.ws + kVerifySlot * (1 + row);
    const u64 old = __hip_atomic_fetch_max(reinterpret_cast<u64*>(slot), key, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old) : "memory");
    __builtin_amdgcn_s_waitcnt(0);
    int last = 0;
    const unsigned chunks = gridDim.x, rows = gridDim.y;
    if (__builtin_amdgcn_atomic_inc32(reinterpret_cast<unsigned*>(slot + 8), chunks - 1, __ATOMIC_RELAXED,
                                      "agent") == chunks - 1)  // this row is complete (its count wrapped)
      last = __builtin_amdgcn_atomic_inc32(reinterpret_cast<unsigned*>(a.ws), rows - 1, __ATOMIC_RELAXED,
                                           "agent") == rows - 1;
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;

  // Last workgroup: collect (and clear) every row's key.
  for (int r = tid; r < a.rows; r += kThreads) {
    const u64 k = __hip_atomic_exchange(reinterpret_cast<u64*>(a.ws + kVerifySlot * (1 + r)), 0ull,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int c = static_cast<int>(0xffffffffu - static_cast<uint32_t>(k));
    s_choice[r] = c;
    a.choice[r] = c;
  }
  __syncthreads();
  if (wave != 0) return;
  // matched[h]: ballot of the nodes 64 h + lane whose token is the target's
  // choice at their parent
  const u64 matched_lo = __ballot(live[0] && tok[0] == s_choice[par[0] + 1]);
  const u64 matched_hi = __ballot(live[1] && tok[1] == s_choice[par[1] + 1]);
  // deepest accepted node (all of its root path matched), lowest index
  // among equally deep ones: the maximum of depth << 8 | (255 - node)
  int node_key = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool accepted = live[h] && (anc_lo[h] & ~matched_lo) == 0ull && (anc_hi[h] & ~matched_hi) == 0ull;
    const int depth_h = __popcll(anc_lo[h]) + __popcll(anc_hi[h]);
    if (accepted) node_key = max(node_key, (depth_h << 8) | (255 - (lane + 64 * h)));
  }
  const int best_node = wave_max_i32(node_key);
  const int depth = best_node >> 8;
  const int last = depth > 0 ? 255 - (best_node & 255) : -1;
  u64 path_lo = 0, path_hi = 0;  // the last node's ancestor set
  if (last >= 0) {
    const int h = last >> 6, l = last & 63;
    path_lo = readlane_u64(h ? anc_lo[1] : anc_lo[0], l);
    path_hi = readlane_u64(h ? anc_hi[1] : anc_hi[0], l);
  }
  // result = [m, bonus, path (root to leaf), -1 ...]: node j on the path goes
  // to position 2 + (number of path nodes below j); ancestors have lower
  // indices, so that is root-to-leaf order.
  if (lane == 0) {
    a.result[0] = depth;
    a.result[1] = s_choice[last + 1];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (live[h]) {
      const int j = lane + 64 * h;
      const u64 below_mask = (1ull << lane) - 1ull;  // bits of this word below j
      const bool on_path = ((h ? path_hi : path_lo) >> lane) & 1ull;
      const int below = h ? __popcll(path_lo) + __popcll(path_hi & below_mask) : __popcll(path_lo & below_mask);
      if (on_path) a.result[2 + below] = j;
      // positions depth .. n-1 hold -1
      if (j >= depth) a.result[2 + j] = -1;
    }
  }
}

}  // namespace

hipError_t launch_tree_verify(const VerifyArgs& a, int32_t dtype, hipStream_t stream) {
  if (a.rows < 1 || a.rows > kMaxVerifyRows || a.vocab < 1) return hipErrorInvalidValue;
  const int64_t epv = dtype == TA_F32 ? 4 : 8;
  const int64_t vecs = (a.vocab + epv - 1) / epv;
  const int64_t per_block = static_cast<int64_t>(kThreads) * kUnroll;
  const dim3 grid(static_cast<unsigned>((vecs + per_block - 1) / per_block), static_cast<unsigned>(a.rows));
  if (dtype == TA_F32)
    hipLaunchKernelGGL(tree_verify_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  else if (dtype == TA_BF16)
    hipLaunchKernelGGL(tree_verify_kernel<__bf16>, grid, dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ta
