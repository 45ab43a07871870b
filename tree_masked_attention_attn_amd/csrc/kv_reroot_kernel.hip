// KV-cache re-root / compaction for gfx950.
//
// SwiftSpec (arXiv 2506.11309), Pith review page, "What carries the argument"
// and "Core claim": after verification the accepted tokens join the verified
// prefix and the surviving tree tokens are packed contiguously after it. In
// slot terms: destination slot dst0 + k receives the row held at src[k]
// (src[k] >= dst0 + k, strictly ascending; the host planner guarantees both),
// in every layer, KV head, K and V. Rows are moved as raw 16-byte words, so
// the result is bit-exact for any element type.
//
// In-place safety. A destination slot can be the source of an EARLIER entry
// (dst0 + k == src[j] with j < k), so a store must not land before that load.
// Hazards only exist within one 16-byte column of one plane. Each workgroup
// owns whole columns of one plane for ALL rows: every thread first loads all
// of its (row, column) items into registers, the workgroup barrier orders
// every load before any store, then the stores run. No scratch memory and no
// cross-workgroup ordering are needed.
//
// The stores are nontemporal: the moved rows stream to HBM instead of
// waiting as dirty L2 lines for the write-back at the kernel's end (an
// 80-layer move of 47 rows, 30.8 MB, measured 15.5 us back to back with
// plain stores and 8.9 us with these).
#include <hip/hip_runtime.h>

#include "launch.h"

namespace ta {
namespace {

constexpr int kThreads = kRerootThreads;
constexpr int kMaxItems = kRerootItemsPerThread;  // (row, 16-B column) items per thread
static_assert(kMaxItems * kThreads < (1 << 17), "item numbers within the reciprocal division's range");
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void kv_reroot_kernel(const RerootArgs a) {
  const int plane = blockIdx.x;            // 0 .. 2*n_planes-1 (K planes, then V planes)
  const int cg = blockIdx.y;               // column group
  char* base = (plane < a.n_planes ? a.k : a.v) +
               (size_t)(plane % a.n_planes) * a.plane_bytes;
  const int cols = a.row_bytes / 16;       // 16-B columns per row
  const int gcols = cols / a.col_groups;   // columns in this group
  const int c0 = cg * gcols;
  const int items = a.n_rows * gcols;

  // item it is (row it / gcols, column it % gcols): the quotient by a
  // multiply with the host's rounded-up reciprocal (exact for it < 2^17 and
  // gcols < 2^15, as here) instead of a division sequence per item
  auto row_of = [&](int it) {
    return gcols == 1 ? it : static_cast<int>(__umulhi(static_cast<uint32_t>(it), a.gcols_rcp));
  };
  uint4 val[kMaxItems];
#pragma unroll
  for (int i = 0; i < kMaxItems; ++i) {
    const int it = threadIdx.x + i * kThreads;
    if (it < items) {
      const int k = row_of(it), c = c0 + it - k * gcols;
      if (a.src[k] != a.dst0 + k)
        val[i] = *reinterpret_cast<const uint4*>(base + (size_t)a.src[k] * a.row_bytes + c * 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMaxItems; ++i) {
    const int it = threadIdx.x + i * kThreads;
    if (it < items) {
      const int k = row_of(it), c = c0 + it - k * gcols;
      if (a.src[k] != a.dst0 + k) {
        // the builtin takes a vector type; the items stay uint4 (an array of
        // vector-typed items compiled to a register copy per use)
        const u32x4 v = {val[i].x, val[i].y, val[i].z, val[i].w};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base + (size_t)(a.dst0 + k) * a.row_bytes + c * 16));
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_reroot(const RerootArgs& a, hipStream_t stream) {
  const int cols = a.row_bytes / 16;
  if (a.col_groups < 1 || cols % a.col_groups != 0 ||
      a.n_rows * (cols / a.col_groups) > kMaxItems * kThreads)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_reroot_kernel, dim3(2 * a.n_planes, a.col_groups), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace ta
