// Wave-wide helpers shared by the verification and expansion kernels.
//
// Reductions over a 64-lane wave use DPP moves inside each 16-lane row
// (quad permutes, then row rotations: every lane ends with its row's
// result) and four readlanes across the rows, so a step costs a couple of
// VALU cycles instead of an LDS round trip of a lane shuffle. Call them with
// every lane of the wave active.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ta {

typedef unsigned long long u64;

// Orderable image of a float: larger float, larger key; -0.0 is taken as
// +0.0, so the two compare equal as they do as floats.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Candidate key of value x at index id: the value first, then the lower
// index (the low word holds ~id). Zero is below every candidate's key (the
// lowest value key, that of -inf, is 0x007fffff), so zero means "none".
__device__ __forceinline__ u64 cand_key(float x, uint32_t id) {
  return (static_cast<u64>(order_key(x)) << 32) | static_cast<u64>(~id);
}

namespace dpp {
constexpr int kXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kRor4 = 0x124;    // row_ror:4
constexpr int kRor8 = 0x128;    // row_ror:8
constexpr int kMirror = 0x140;      // row_mirror: lane i of a row reads lane 15 - i
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i of an 8-lane half reads lane 7 - i
constexpr int kBcast15 = 0x142; // row_bcast:15 (lane 15 of a row to the next row)
constexpr int kBcast31 = 0x143; // row_bcast:31 (lane 31 to rows 2 and 3)
}  // namespace dpp

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ unsigned dpp_u32(unsigned v) {
  // rows outside ROWS keep their own value
  return static_cast<unsigned>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, ROWS, 0xF, false));
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ u64 dpp_u64(u64 v) {
  return (static_cast<u64>(dpp_u32<CTRL, ROWS>(static_cast<unsigned>(v >> 32))) << 32) |
         dpp_u32<CTRL, ROWS>(static_cast<unsigned>(v));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

__device__ __forceinline__ u64 readlane_u64(u64 v, int lane) {
  return (static_cast<u64>(static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), lane)))
          << 32) |
         static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __uint_as_float(static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v)), lane)));
}

// Maximum over the wave, returned to every lane (a uniform value): a
// butterfly inside each row, then the row broadcasts carry the running
// maximum on to lane 63. Each step is one max with a DPP operand.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t k) {
  // lanes of rows outside ROWS see 0, the identity of the max
  return max(k, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(k), CTRL, ROWS, 0xF, false)));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
  k = dpp_max_u32<dpp::kXor1>(k);
  k = dpp_max_u32<dpp::kXor2>(k);
  k = dpp_max_u32<dpp::kRor4>(k);
  k = dpp_max_u32<dpp::kRor8>(k);
  k = dpp_max_u32<dpp::kBcast15, 0xA>(k);
  k = dpp_max_u32<dpp::kBcast31, 0xC>(k);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(k), 63));
}

// 64-bit maximum as two 32-bit ones: the high words, then the low words of
// the lanes that hold the highest high word.
__device__ __forceinline__ u64 wave_max_u64(u64 k) {
  const uint32_t hi = wave_max_u32(static_cast<uint32_t>(k >> 32));
  const uint32_t lo = wave_max_u32(static_cast<uint32_t>(k >> 32) == hi ? static_cast<uint32_t>(k) : 0u);
  return (static_cast<u64>(hi) << 32) | lo;
}

// Float maximum and sum over the wave, returned to every lane: DPP steps
// inside each 16-lane row, then the four rows' results (a fixed order, so
// the sum is the same on every call).
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<dpp::kXor1>(x));
  x = fmaxf(x, dpp_f32<dpp::kXor2>(x));
  x = fmaxf(x, dpp_f32<dpp::kRor4>(x));
  x = fmaxf(x, dpp_f32<dpp::kRor8>(x));
  return fmaxf(fmaxf(readlane_f32(x, 0), readlane_f32(x, 16)), fmaxf(readlane_f32(x, 32), readlane_f32(x, 48)));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  x += dpp_f32<dpp::kXor1>(x);
  x += dpp_f32<dpp::kXor2>(x);
  x += dpp_f32<dpp::kRor4>(x);
  x += dpp_f32<dpp::kRor8>(x);
  return (readlane_f32(x, 0) + readlane_f32(x, 16)) + (readlane_f32(x, 32) + readlane_f32(x, 48));
}

// Maximum of non-negative ints over the wave.
__device__ __forceinline__ int wave_max_i32(int k) {
  return static_cast<int>(wave_max_u32(static_cast<uint32_t>(k)));
}

}  // namespace ta
