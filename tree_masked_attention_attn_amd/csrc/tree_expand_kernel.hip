// Maximum-likelihood expansion step for gfx950: the k best (leaf, token)
// children of a draft tree's frontier, in one launch.
//
// SwiftSpec (arXiv 2506.11309), Pith review page, "Assumptions & free
// parameters": the draft tree grows by maximum likelihood, a path scoring the
// sum of its tokens' log-softmax probabilities, with expansion width w = 8.
// For frontier leaf i with path score s[i] and draft logits x[i] over the
// vocabulary, every token t is a candidate child with score
// s[i] + x[i][t] - logsumexp(x[i]); the k best become the new nodes. Within a
// leaf the candidates rank by logit (lower token id first on ties), which is
// their slot; equal scores go to the lower leaf, then the lower slot; the
// output lists the new nodes by (leaf, slot).
//
// Work split (HBM-bound: each logit is read once). The grid is (chunk of
// 4096 logits, leaf). A workgroup computes its chunk's (max, sum of exp) and
// its k best (logit, token) keys, stores them in its slot of the workspace
// (write-through, so that another XCD reads them from memory) and counts in
// on its leaf. The leaf's last chunk (its wrapping count) merges the chunks
// into the leaf's logsumexp and its k best tokens, turns them into fp32
// scores, publishes them and counts the leaf in; the last leaf's last chunk
// selects the k best of all leaves and writes them. Each count per address
// takes a leaf's chunks or the leaves, never the whole grid.
//
// Selection without serial rounds. Every k-best step works on lists of L
// keys (L = 8 or 16, at least k), sorted largest first and held in
// registers. A thread sorts its own keys with a bitonic network; two sorted
// lists a and b combine into their L best in one step, since the pairwise
// maxima max(a[i], b[L-1-i]) are exactly those L keys in bitonic order, which
// a bitonic merge sorts. Taking b from another lane by a DPP move, six such
// steps (row mirror, half-row mirror, two quad swaps, two row broadcasts)
// merge all 64 lanes' lists into lane 63's. Keys are unique (they carry the
// token, or leaf and slot), so the result is the same set in the same order
// as k rounds of "take the largest" would give. For bf16 logits the leaf
// merge works on 32-bit keys (value, chunk, slot in the chunk's list), the
// token read back from that list. The final choice among w * k <= 64
// candidates is by rank: each lane holds one and counts the keys above its
// own, with no dependent chain of merges.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "launch.h"
#include "tree_attn.h"
#include "wave_ops.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;                 // logits per thread
constexpr int kChunk = kThreads * kPerThread;  // logits per workgroup
constexpr int kWriteThrough = 16;              // cache policy of workspace traffic (sc1)
constexpr int kKeysAt = 16;                    // a chunk slot: (max, sum), pad, then k keys (16-byte loads)
static_assert(kKeysAt + 8 * kExpandMaxK <= kExpandChunkSlot, "chunk slot size");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
static_assert(kChunk == kExpandChunk, "chunk size shared with the host");

// (max, sum of exp(x - max)) of the union of two sets; (-inf, 0) is empty.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float a = m == kNegInf ? 0.f : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
  const float b = m2 == kNegInf ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - M) * kLog2e);
  m = M;
  s = a + b;
}

// A logsumexp over a wave takes the wave's maximum first and sums
// exp(x - max) after it (wave_max_f32, wave_sum_f32), so no exponential sits
// on the reduction's dependent chain.
// (max, sum of exp(x - max)) over the wave from every lane's own pair.
__device__ __forceinline__ void lse_wave(float& m, float& s) {
  const float M = wave_max_f32(m);
  s = wave_sum_f32(m == kNegInf ? 0.f : s * __builtin_amdgcn_exp2f((m - M) * kLog2e));
  m = M;
}

// Keys inside one chunk. bf16 logits: the top 16 bits of the value's
// orderable image (the low 16 are fixed by the sign) and the lower
// in-chunk index (12 bits) fit one 32-bit word, so each selection round is
// one 32-bit wave maximum; fp32 logits keep 64-bit (value, ~token) keys.
template <typename T>
using ChunkKey = std::conditional_t<std::is_same_v<T, float>, u64, uint32_t>;

template <typename T>
__device__ __forceinline__ ChunkKey<T> chunk_key(float f, uint32_t id, int local) {
  if constexpr (std::is_same_v<T, float>)
    return cand_key(f, id);
  else
    return (order_key(f) & 0xffff0000u) | static_cast<uint32_t>(kChunk - 1 - local);
}

// The 16-bit orderable images of the two bf16 values in x (low half, high
// half), as chunk_key takes them: a negative value's bits inverted, a
// non-negative one's sign bit set, -0.0 taken as +0.0. Packed 16-bit integer
// operations handle both halves at once.
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair_images(uint32_t x) {
  const uint32_t mag = x & 0x7fff7fffu;
  const i16x2 neg = __builtin_bit_cast(i16x2, x) >> 15;  // all ones where the sign bit is set
  const i16x2 nz = __builtin_bit_cast(i16x2, __builtin_bit_cast(u16x2, mag) + u16x2{0x7fff, 0x7fff}) >>
                   15;  // all ones where the magnitude is not zero
  return (mag | 0x80008000u) ^ __builtin_bit_cast(uint32_t, neg & nz);
}

// A bf16 chunk key's logit and token (chunk `chunk`): the value's orderable
// image is its top half, the low half being all ones for a negative value
// and zero otherwise.
__device__ __forceinline__ float chunk_key_value(uint32_t k) {
  const uint32_t hi = k & 0xffff0000u;
  return key_value(hi | ((hi & 0x80000000u) ? 0u : 0xffffu));
}
__device__ __forceinline__ int chunk_key_token(uint32_t k, int chunk) {
  return chunk * kChunk + (kChunk - 1 - static_cast<int>(k & 0xfffu));
}

// Leaf-level key of slot r of chunk c's list (bf16): the value's 16-bit
// image, then the lower chunk, then the lower slot. Chunks cover ascending
// token ranges and a chunk's list is in (value, lower token) order, so this
// 32-bit key orders candidates exactly as (value, lower token) does; the
// token is read back from the chunk's list. Zero stays zero (an empty slot);
// a real key is never zero since 64 - c >= 1.
__device__ __forceinline__ uint32_t leaf_key(uint32_t ck, int c, int r) {
  return ck == 0 ? 0u : (ck & 0xffff0000u) | (static_cast<uint32_t>(64 - c) << 4) | static_cast<uint32_t>(15 - r);
}
static_assert(kExpandMaxChunks <= 64 && kExpandMaxK <= 16, "leaf key fields");

template <typename K>
__device__ __forceinline__ K kmax(K a, K b) { return a > b ? a : b; }
template <typename K>
__device__ __forceinline__ K kmin(K a, K b) { return a > b ? b : a; }

// a, b <- the larger, the smaller (32-bit keys: a max and a min; 64-bit
// keys: one comparison selecting both halves of both)
__device__ __forceinline__ void cas(uint32_t& a, uint32_t& b) {
  const uint32_t hi = kmax(a, b), lo = kmin(a, b);
  a = hi;
  b = lo;
}
__device__ __forceinline__ void cas(u64& a, u64& b) {
  const bool gt = a > b;
  const u64 hi = gt ? a : b, lo = gt ? b : a;
  a = hi;
  b = lo;
}

// r[0..N), a bitonic sequence, into descending order (half-cleaners at
// distances N/2, .., 1).
template <int N, typename K, int M>
__device__ __forceinline__ void bitonic_merge_desc(K (&r)[M]) {
  static_assert(N <= M && (N & (N - 1)) == 0, "power of two");
#pragma unroll
  for (int d = N / 2; d >= 1; d /= 2)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & d) == 0) cas(r[i], r[i + d]);
}

// r[0..N) into descending order: bitonic sort, blocks of each size sorted
// in alternating directions so that each pair of them forms a bitonic run.
template <int N, int OFF, typename K, int M>
__device__ __forceinline__ void bitonic_sort_desc(K (&r)[M]) {
  static_assert(OFF + N <= M && (N & (N - 1)) == 0, "power of two");
#pragma unroll
  for (int size = 2; size <= N; size *= 2)
#pragma unroll
    for (int d = size / 2; d >= 1; d /= 2)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ d;
        if (j > i) {
          if ((i & size) == 0) cas(r[OFF + i], r[OFF + j]);
          else cas(r[OFF + j], r[OFF + i]);
        }
      }
}

// A key of the lane that DPP control CTRL selects (lanes of rows outside
// ROWS get their own).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_key(uint32_t x) {
  return dpp_u32<CTRL, ROWS>(x);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ u64 dpp_key(u64 x) {
  return dpp_u64<CTRL, ROWS>(x);
}

// This lane's sorted list and the CTRL-selected lane's -> their L best, sorted.
template <int CTRL, int ROWS, int L, typename K>
__device__ __forceinline__ void merge_lanes(K (&r)[L]) {
  K c[L];
#pragma unroll
  for (int i = 0; i < L; ++i) c[i] = kmax(r[i], dpp_key<CTRL, ROWS>(r[L - 1 - i]));
  bitonic_merge_desc<L>(c);
#pragma unroll
  for (int i = 0; i < L; ++i) r[i] = c[i];
}

// The L best keys of the sorted lists of lanes 0 .. n-1 (the other lanes'
// lists empty), sorted, in the lane returned. The half-row mirror and two
// quad swaps leave in every lane of an 8-lane half the best of that half,
// with the row mirror first of a 16-lane row (each step pairs lanes whose
// sets are disjoint); the row broadcasts then fold row 0 into row 1, row 2
// into row 3, and row 1 into row 3. n is the same in every lane.
template <int L, typename K>
__device__ __forceinline__ int wave_top(K (&r)[L], int n) {
  if (n > 8) merge_lanes<dpp::kMirror, 0xF>(r);
  merge_lanes<dpp::kHalfMirror, 0xF>(r);
  merge_lanes<dpp::kXor2, 0xF>(r);
  merge_lanes<dpp::kXor1, 0xF>(r);
  if (n <= 16) return 0;
  merge_lanes<dpp::kBcast15, 0xA>(r);
  if (n <= 32) return 31;
  merge_lanes<dpp::kBcast31, 0xC>(r);
  return 63;
}

// Lane `src`'s key r[i], for every lane.
__device__ __forceinline__ uint32_t readlane_key(uint32_t x, int src) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), src));
}
__device__ __forceinline__ u64 readlane_key(u64 x, int src) { return readlane_u64(x, src); }

// Element i of lane `src`'s list, into lane i (i < n): a list spread over lanes.
template <int L, typename K>
__device__ __forceinline__ K spread_list(const K (&r)[L], int src, int lane, int n) {
  K mine = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (i < n) {
      const K v = readlane_key(r[i], src);
      if (lane == i) mine = v;
    }
  }
  return mine;
}

// The L best of a thread's 16 keys, sorted: both halves sorted, then their
// pairwise maxima (the 8 best, bitonic) merged; for L = 16 all of them.
template <int L, typename K>
__device__ __forceinline__ void thread_top(K (&key)[kPerThread], K (&top)[L]) {
  static_assert(kPerThread == 16 && (L == 8 || L == 16), "list sizes");
  if constexpr (L == 16) {
    bitonic_sort_desc<16, 0>(key);
#pragma unroll
    for (int i = 0; i < 16; ++i) top[i] = key[i];
  } else {
    bitonic_sort_desc<8, 0>(key);
    bitonic_sort_desc<8, 8>(key);
#pragma unroll
    for (int i = 0; i < 8; ++i) top[i] = kmax(key[i], key[15 - i]);
    bitonic_merge_desc<8>(top);
  }
}

template <typename T, int L>
__global__ __launch_bounds__(kThreads) void tree_expand_kernel(const ExpandArgs a) {
  using CK = ChunkKey<T>;
  constexpr int EPV = 16 / sizeof(T);         // logits per 16-byte vector
  constexpr int NV = kPerThread / EPV;        // vectors per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int K = a.k;  // <= L
  const T* x = static_cast<const T*>(a.logits) + static_cast<size_t>(row) * a.row_stride;
  const int64_t full_vecs = a.vocab / EPV;
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(a.ws, 0, a.ws_bytes, 0x00020000);
  // loaded by every workgroup with the logits, its latency hidden there,
  // though only the leaf's last chunk uses it
  const float s_leaf = a.path_scores[row];

  // Thread tid reads vectors tid, tid + 256, .. of the chunk: whole vectors
  // with 16-byte loads; a vector that would run past the vocabulary (only
  // in the last chunk) is never loaded whole but filled element by element,
  // -inf past the end. The per-logit work below is then free of branches
  // (one branch per logit measured 1.3 us per call).
  u32x4 buf[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = static_cast<int64_t>(chunk) * (kChunk / EPV) + j * kThreads + tid;
    if (vi < full_vecs) buf[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + vi);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = static_cast<int64_t>(chunk) * (kChunk / EPV) + j * kThreads + tid;
    if (vi >= full_vecs) {
      T tail[EPV];
#pragma unroll
      for (int t = 0; t < EPV; ++t) {
        const int64_t id = vi * EPV + t;
        tail[t] = id < a.vocab ? x[id] : static_cast<T>(kNegInf);
      }
      buf[j] = __builtin_bit_cast(u32x4, tail);
    }
  }
  float v[kPerThread];
  CK key[kPerThread];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = static_cast<int64_t>(chunk) * (kChunk / EPV) + j * kThreads + tid;
    if constexpr (std::is_same_v<T, float>) {
      const T* e = reinterpret_cast<const T*>(&buf[j]);
#pragma unroll
      for (int t = 0; t < EPV; ++t) {
        const int64_t id = vi * EPV + t;
        const float f = e[t];
        v[j * EPV + t] = f;
        key[j * EPV + t] = id < a.vocab ? chunk_key<T>(f, static_cast<uint32_t>(id),
                                                       static_cast<int>(id - static_cast<int64_t>(chunk) * kChunk))
                                        : CK{0};
      }
    } else {
      // two logits per 32-bit word: both keys' value images at once, then
      // each with its in-chunk index; slots past the vocabulary (only in a
      // vector that runs past it) are emptied afterwards
      const int local = (j * kThreads + tid) * EPV;  // in-chunk index of the vector's first logit
#pragma unroll
      for (int q = 0; q < EPV / 2; ++q) {
        const uint32_t x = buf[j][q];
        const uint32_t k2 = bf16_pair_images(x);
        v[j * EPV + 2 * q] = __uint_as_float(x << 16);
        v[j * EPV + 2 * q + 1] = __uint_as_float(x & 0xffff0000u);
        key[j * EPV + 2 * q] = (k2 << 16) | static_cast<uint32_t>(kChunk - 1 - local - 2 * q);
        key[j * EPV + 2 * q + 1] = (k2 & 0xffff0000u) | static_cast<uint32_t>(kChunk - 2 - local - 2 * q);
      }
      if (vi >= full_vecs) {
#pragma unroll
        for (int t = 0; t < EPV; ++t)
          if (vi * EPV + t >= a.vocab) key[j * EPV + t] = 0;
      }
    }
  }

  // The wave's (max, sum of exp): the maximum first.
  float m = kNegInf;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) m = fmaxf(m, v[i]);
  m = wave_max_f32(m);
  float s = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) s += __builtin_amdgcn_exp2f((v[i] - m) * kLog2e);
  }
  s = wave_sum_f32(s);

  // The wave's L best keys, then the workgroup's (wave 0, lane 0).
  __shared__ CK s_key[4][L];
  __shared__ float s_m[4], s_s[4];
  {
    CK top[L];
    thread_top<L>(key, top);
    if (lane == wave_top<L>(top, 64)) {
#pragma unroll
      for (int i = 0; i < L; ++i) s_key[wave][i] = top[i];
    }
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_s[wave] = s;
  }
  __syncthreads();
  if (wave != 0) return;

  CK c4[L];
#pragma unroll
  for (int i = 0; i < L; ++i) c4[i] = lane < 4 ? s_key[lane][i] : CK{0};
  merge_lanes<dpp::kXor1, 0xF>(c4);
  merge_lanes<dpp::kXor2, 0xF>(c4);  // lane 0: the chunk's L best
  const CK mine = spread_list<L>(c4, 0, lane, K);  // lane i < K: the chunk's key i
  float cm = s_m[0], cs = s_s[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) lse_merge(cm, cs, s_m[w], s_s[w]);

  const int cslot = kExpandChunkBase + (row * kExpandMaxChunks + chunk) * kExpandChunkSlot;
  if (lane < K) {
    if constexpr (std::is_same_v<T, float>)
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, mine), ws, cslot + kKeysAt + 8 * lane, 0,
                                            kWriteThrough);
    else
      __builtin_amdgcn_raw_buffer_store_b32(mine, ws, cslot + kKeysAt + 4 * lane, 0, kWriteThrough);
  }
  if (lane == 0)
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, make_float2(cm, cs)), ws, cslot, 0,
                                          kWriteThrough);
  // The stores complete before the count announces them.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  int last = 0;
  if (lane == 0)
    last = __builtin_amdgcn_atomic_inc32(reinterpret_cast<unsigned*>(a.ws + kExpandRowCount * (1 + row)),
                                         a.chunks - 1, __ATOMIC_RELAXED, "agent") == static_cast<unsigned>(a.chunks - 1);
  if (!__builtin_amdgcn_readfirstlane(last)) return;

  // The leaf's last chunk: lane c reads chunk c's (max, sum) and its K keys
  // (device-scope loads: they see memory as the count did), a sorted list.
  float lm = kNegInf, ls = 0.f;
  float score = 0.f;
  int tok = -1;
  if constexpr (std::is_same_v<T, float>) {
    u64 kk[L];
#pragma unroll
    for (int r = 0; r < L; ++r) kk[r] = 0;
    if (lane < a.chunks) {
      const int sl = kExpandChunkBase + (row * kExpandMaxChunks + lane) * kExpandChunkSlot;
      const float2 ms = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(ws, sl, 0, kWriteThrough));
      lm = ms.x;
      ls = ms.y;
#pragma unroll
      for (int q = 0; q < L / 2; ++q) {
        if (2 * q < K) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ws, sl + kKeysAt + 16 * q, 0, kWriteThrough);
          kk[2 * q] = (static_cast<u64>(v.y) << 32) | v.x;
          if (2 * q + 1 < K) kk[2 * q + 1] = (static_cast<u64>(v.w) << 32) | v.z;
        }
      }
    }
    lse_wave(lm, ls);
    const int at2 = wave_top<L>(kk, a.chunks);  // lane at2: the leaf's L best
    const u64 rk = spread_list<L>(kk, at2, lane, K);
    score = key_value(static_cast<uint32_t>(rk >> 32));
    tok = rk != 0 ? static_cast<int>(~static_cast<uint32_t>(rk)) : -1;
  } else {
    // 32-bit leaf keys (value, chunk, slot); the chunks' lists stay in LDS
    // for the token look-up.
    __shared__ uint32_t s_ck[kExpandMaxChunks][L];
    uint32_t lk[L];
#pragma unroll
    for (int r = 0; r < L; ++r) lk[r] = 0;
    if (lane < a.chunks) {
      const int sl = kExpandChunkBase + (row * kExpandMaxChunks + lane) * kExpandChunkSlot;
      const float2 ms = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(ws, sl, 0, kWriteThrough));
      lm = ms.x;
      ls = ms.y;
#pragma unroll
      for (int q = 0; q < L / 4; ++q) {
        if (4 * q < K) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ws, sl + kKeysAt + 16 * q, 0, kWriteThrough);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q + e;
            if (r < K) {
              s_ck[lane][r] = v[e];
              lk[r] = leaf_key(v[e], lane, r);
            }
          }
        }
      }
    }
    lse_wave(lm, ls);
    const int at2 = wave_top<L>(lk, a.chunks);  // lane at2: the leaf's L best
    const uint32_t rk = spread_list<L>(lk, at2, lane, K);
    // the LDS writes above come before these reads in every lane's program
    // order; LDS serves one wave's accesses in issue order
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (rk != 0) {
      const int c = 64 - static_cast<int>((rk >> 4) & 127u), r = 15 - static_cast<int>(rk & 15u);
      const uint32_t ck = s_ck[c][r];
      score = chunk_key_value(ck);
      tok = chunk_key_token(ck, c);
    }
  }
  const float log_sum = __logf(ls);  // logsumexp = lm + log_sum
  const int rslot = kExpandRowBase + row * kExpandRowSlot;
  if (lane < K) {
    // slot `lane` of this leaf: (score, token), or token -1 when the leaf
    // has fewer than K tokens
    const float sc = s_leaf + ((score - lm) - log_sum);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(sc), static_cast<unsigned>(tok)}, ws,
                                          rslot + 8 * lane, 0, kWriteThrough);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  last = 0;
  if (lane == 0)
    last = __builtin_amdgcn_atomic_inc32(reinterpret_cast<unsigned*>(a.ws), a.w - 1, __ATOMIC_RELAXED,
                                         "agent") == static_cast<unsigned>(a.w - 1);
  if (!__builtin_amdgcn_readfirstlane(last)) return;

  // The last leaf. Candidate (leaf i, slot r) has the key (score, then the
  // lower leaf, then the lower slot); zero for an empty slot, below every
  // real key. At least K candidates are real (k <= w * vocab), and real keys
  // are unique.
  const int n = a.w * K;
  if (n <= 64) {
    // One candidate per lane, lane = leaf * K + slot: a candidate is chosen
    // iff fewer than K keys exceed its own, and the chosen lanes, in lane
    // order, are already in (leaf, slot) order.
    __shared__ u64 s_hk[64];
    int leaf = 0, slot = 0, ctok = -1;
    float csc = 0.f;
    u64 hk = 0;
    if (lane < n) {
      leaf = lane / K;
      slot = lane - leaf * K;
      const u32x2 p = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(ws, kExpandRowBase + leaf * kExpandRowSlot + 8 * slot, 0,
                                                      kWriteThrough));
      csc = __uint_as_float(p.x);
      ctok = static_cast<int>(p.y);
      hk = ctok >= 0 ? (static_cast<u64>(order_key(csc)) << 32) |
                           static_cast<u64>(~static_cast<uint32_t>((leaf << 8) | slot))
                     : 0ull;
    }
    s_hk[lane] = hk;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    int above = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) above += s_hk[j] > hk ? 1 : 0;
    const bool chosen = lane < n && hk != 0 && above < K;
    const u64 sel = __ballot(chosen);
    if (chosen) {
      const int pos = __popcll(sel & ((1ull << lane) - 1ull));
      a.leaf_out[pos] = leaf;
      a.token_out[pos] = ctok;
      a.score_out[pos] = csc;
    }
    return;
  }

  // More candidates than lanes: lane l holds leaf l's K (score, token) in
  // slot order, a sorted list, and the lists are merged.
  __shared__ float s_sc[kExpandMaxRows][L];
  __shared__ int s_tk[kExpandMaxRows][L];
  u64 hk[L];
#pragma unroll
  for (int r = 0; r < L; ++r) hk[r] = 0;
  if (lane < a.w) {
#pragma unroll
    for (int r = 0; r < L; ++r) {
      if (r < K) {
        const u32x2 p = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(ws, kExpandRowBase + lane * kExpandRowSlot + 8 * r, 0,
                                                        kWriteThrough));
        const float sc = __uint_as_float(p.x);
        const int tk = static_cast<int>(p.y);
        s_sc[lane][r] = sc;
        s_tk[lane][r] = tk;
        hk[r] = tk >= 0 ? (static_cast<u64>(order_key(sc)) << 32) |
                              static_cast<u64>(~static_cast<uint32_t>((lane << 8) | r))
                        : 0ull;
      }
    }
  }
  const int at3 = wave_top<L>(hk, a.w);  // lane at3: the K best of all leaves
  const uint32_t who = ~static_cast<uint32_t>(spread_list<L>(hk, at3, lane, K));  // (leaf << 8) | slot
  int out_leaf = 0, out_slot = 0, out_tok = 0;
  float out_score = 0.f;
  if (lane < K) {
    out_leaf = static_cast<int>(who >> 8);
    out_slot = static_cast<int>(who & 255u);
    out_tok = s_tk[out_leaf][out_slot];
    out_score = s_sc[out_leaf][out_slot];
  }
  // List the K new nodes by (leaf, slot).
  const int mykey = (out_leaf << 8) | out_slot;
  int pos = 0;
#pragma unroll
  for (int j = 0; j < kExpandMaxK; ++j) {
    if (j < K) pos += __builtin_amdgcn_readlane(mykey, j) < mykey ? 1 : 0;
  }
  if (lane < K) {
    a.leaf_out[pos] = out_leaf;
    a.token_out[pos] = out_tok;
    a.score_out[pos] = out_score;
  }
}

}  // namespace

hipError_t launch_tree_expand(const ExpandArgs& a, int32_t dtype, hipStream_t stream) {
  if (a.w < 1 || a.w > kExpandMaxRows || a.k < 1 || a.k > kExpandMaxK || a.chunks < 1 ||
      a.chunks > kExpandMaxChunks || static_cast<int64_t>(a.chunks) * kChunk < a.vocab)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.chunks), static_cast<unsigned>(a.w));
  // lists of 8 keys for k <= 8, of 16 above
  const bool small = a.k <= 8;
  if (dtype == TA_F32) {
    if (small) hipLaunchKernelGGL((tree_expand_kernel<float, 8>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((tree_expand_kernel<float, 16>), grid, dim3(kThreads), 0, stream, a);
  } else if (dtype == TA_BF16) {
    if (small) hipLaunchKernelGGL((tree_expand_kernel<__bf16, 8>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((tree_expand_kernel<__bf16, 16>), grid, dim3(kThreads), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ta
