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
// its k best (logit, token) keys: each wave extracts k winners with shuffles
// only, then one wave merges the four waves' 4k. It stores them in its slot
// of the workspace (write-through, so that another XCD reads them from
// memory) and counts in on its leaf. The leaf's last chunk (its wrapping
// count) merges the chunks into the leaf's logsumexp and its k best tokens,
// turns them into fp32 scores, publishes them and counts the leaf in; the
// last leaf's last chunk selects the k best of all leaves and writes them.
// Each count per address takes a leaf's chunks or the leaves, never the
// whole grid.
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

// (max, sum) of the whole wave, returned to every lane.
__device__ __forceinline__ void lse_wave(float& m, float& s) {
  lse_merge(m, s, dpp_f32<dpp::kXor1>(m), dpp_f32<dpp::kXor1>(s));
  lse_merge(m, s, dpp_f32<dpp::kXor2>(m), dpp_f32<dpp::kXor2>(s));
  lse_merge(m, s, dpp_f32<dpp::kRor4>(m), dpp_f32<dpp::kRor4>(s));
  lse_merge(m, s, dpp_f32<dpp::kRor8>(m), dpp_f32<dpp::kRor8>(s));
  float m0 = readlane_f32(m, 0), s0 = readlane_f32(s, 0);
  lse_merge(m0, s0, readlane_f32(m, 16), readlane_f32(s, 16));
  lse_merge(m0, s0, readlane_f32(m, 32), readlane_f32(s, 32));
  lse_merge(m0, s0, readlane_f32(m, 48), readlane_f32(s, 48));
  m = m0;
  s = s0;
}

template <typename T>
__device__ __forceinline__ float to_float(T x) {
  if constexpr (std::is_same_v<T, float>)
    return x;
  else
    return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) << 16);
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

// The 64-bit (value, ~token) key of a chunk key (zero stays zero).
template <typename T>
__device__ __forceinline__ u64 global_key(ChunkKey<T> k, int chunk) {
  if constexpr (std::is_same_v<T, float>) {
    return k;
  } else {
    if (k == 0) return 0ull;
    const uint32_t hi = k & 0xffff0000u;
    const uint32_t ok = hi | ((hi & 0x80000000u) ? 0u : 0xffffu);  // the orderable image's low half
    const uint32_t id = static_cast<uint32_t>(chunk * kChunk + (kChunk - 1 - static_cast<int>(k & 0xfffu)));
    return (static_cast<u64>(ok) << 32) | static_cast<u64>(~id);
  }
}

__device__ __forceinline__ u64 wave_max_key(u64 k) { return wave_max_u64(k); }
__device__ __forceinline__ uint32_t wave_max_key(uint32_t k) { return wave_max_u32(k); }

template <typename T>
__global__ __launch_bounds__(kThreads) void tree_expand_kernel(const ExpandArgs a) {
  using CK = ChunkKey<T>;
  constexpr int EPV = 16 / sizeof(T);         // logits per 16-byte vector
  constexpr int NV = kPerThread / EPV;        // vectors per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int K = a.k;
  const T* x = static_cast<const T*>(a.logits) + static_cast<size_t>(row) * a.row_stride;
  const int64_t full_vecs = a.vocab / EPV;
  const float s_leaf = a.path_scores[row];  // used by the leaf's last chunk
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(a.ws, 0, a.ws_bytes, 0x00020000);

  // Thread tid reads vectors tid, tid + 256, .. of the chunk: whole vectors
  // with 16-byte loads, a ragged tail element by element (a vector that
  // would run past the vocabulary is never loaded).
  u32x4 buf[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = static_cast<int64_t>(chunk) * (kChunk / EPV) + j * kThreads + tid;
    if (vi < full_vecs) buf[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + vi);
  }
  float v[kPerThread];
  CK key[kPerThread];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = static_cast<int64_t>(chunk) * (kChunk / EPV) + j * kThreads + tid;
    const T* e = reinterpret_cast<const T*>(&buf[j]);
#pragma unroll
    for (int t = 0; t < EPV; ++t) {
      const int64_t id = vi * EPV + t;
      float f = kNegInf;
      bool ok = false;
      if (vi < full_vecs) {
        f = to_float(e[t]);
        ok = true;
      } else if (id < a.vocab) {
        f = to_float(x[id]);
        ok = true;
      }
      v[j * EPV + t] = f;
      key[j * EPV + t] =
          ok ? chunk_key<T>(f, static_cast<uint32_t>(id), static_cast<int>(id - static_cast<int64_t>(chunk) * kChunk))
             : CK{0};
    }
  }

  // This thread's (max, sum of exp).
  float m = kNegInf;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) m = fmaxf(m, v[i]);
  float s = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) s += __builtin_amdgcn_exp2f((v[i] - m) * kLog2e);
  }
  lse_wave(m, s);

  // The wave's K best keys: K rounds of a wave maximum over each lane's best
  // key below the last winner (keys are unique: they hold the token id).
  auto best_below = [&](CK lim) {
    CK b = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) b = (key[i] < lim && key[i] > b) ? key[i] : b;
    return b;
  };
  __shared__ CK s_key[4][kExpandMaxK];
  __shared__ float s_m[4], s_s[4];
  // The lane's best and second-best keys: a winner moves on to its second
  // and only re-scans its keys when that one is taken too.
  CK cand = 0, alt = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const CK q = key[i];
    alt = q > cand ? cand : (q > alt ? q : alt);
    cand = q > cand ? q : cand;
  }
#pragma unroll
  for (int r = 0; r < kExpandMaxK; ++r) {
    if (r < K) {
      const CK w = wave_max_key(cand);
      if (lane == 0) s_key[wave][r] = w;
      if (cand == w && w != 0) {
        cand = alt != 0 ? alt : best_below(w);
        alt = 0;
      }
    }
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_s[wave] = s;
  }
  __syncthreads();
  if (wave != 0) return;

  // Wave 0: the chunk's K best of the four waves' 4K, and its (max, sum).
  CK c4 = lane < 4 * K ? s_key[lane / K][lane % K] : CK{0};
  CK mine_c = 0;  // lane r keeps round r's winner
#pragma unroll
  for (int r = 0; r < kExpandMaxK; ++r) {
    if (r < K) {
      const CK w = wave_max_key(c4);
      if (lane == r) mine_c = w;
      if (c4 == w) c4 = 0;
    }
  }
  const u64 mine = global_key<T>(mine_c, chunk);
  float cm = s_m[0], cs = s_s[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) lse_merge(cm, cs, s_m[w], s_s[w]);

  const int cslot = kExpandChunkBase + (row * kExpandMaxChunks + chunk) * kExpandChunkSlot;
  if (lane < K)
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, mine), ws, cslot + 8 + 8 * lane, 0,
                                          kWriteThrough);
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
  // (device-scope loads: they see memory as the count did).
  float lm = kNegInf, ls = 0.f;
  u64 kk[kExpandMaxK];
#pragma unroll
  for (int r = 0; r < kExpandMaxK; ++r) kk[r] = 0;
  if (lane < a.chunks) {
    const int sl = kExpandChunkBase + (row * kExpandMaxChunks + lane) * kExpandChunkSlot;
    const float2 ms = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(ws, sl, 0, kWriteThrough));
    lm = ms.x;
    ls = ms.y;
#pragma unroll
    for (int r = 0; r < kExpandMaxK; ++r)
      if (r < K) kk[r] = __builtin_bit_cast(u64, __builtin_amdgcn_raw_buffer_load_b64(ws, sl + 8 + 8 * r, 0, kWriteThrough));
  }
  lse_wave(lm, ls);
  const float log_sum = __logf(ls);  // logsumexp = lm + log_sum
  // K rounds over the chunks' sorted lists: the lane holding the winner
  // drops its head.
  u64 rk = 0;
#pragma unroll
  for (int r = 0; r < kExpandMaxK; ++r) {
    if (r < K) {
      const u64 w = wave_max_u64(kk[0]);
      if (lane == r) rk = w;
      if (kk[0] == w && w != 0) {
#pragma unroll
        for (int i = 0; i + 1 < kExpandMaxK; ++i) kk[i] = kk[i + 1];
        kk[kExpandMaxK - 1] = 0;
      }
    }
  }
  const int rslot = kExpandRowBase + row * kExpandRowSlot;
  if (lane < K) {
    // slot `lane` of this leaf: (score, token), or token -1 when the leaf
    // has fewer than K tokens
    const float score = s_leaf + ((key_value(static_cast<uint32_t>(rk >> 32)) - lm) - log_sum);
    const int tok = rk != 0 ? static_cast<int>(~static_cast<uint32_t>(rk)) : -1;
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(score), static_cast<unsigned>(tok)}, ws,
                                          rslot + 8 * lane, 0, kWriteThrough);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  last = 0;
  if (lane == 0)
    last = __builtin_amdgcn_atomic_inc32(reinterpret_cast<unsigned*>(a.ws), a.w - 1, __ATOMIC_RELAXED,
                                         "agent") == static_cast<unsigned>(a.w - 1);
  if (!__builtin_amdgcn_readfirstlane(last)) return;

  // The last leaf: lane l holds leaf l's K (score, token) in slot order; K
  // rounds pick the best head (score, then the lower leaf, then the lower
  // slot), whose lane drops it.
  float sc[kExpandMaxK];
  int tk[kExpandMaxK];
#pragma unroll
  for (int r = 0; r < kExpandMaxK; ++r) {
    sc[r] = kNegInf;
    tk[r] = -1;
  }
  if (lane < a.w) {
#pragma unroll
    for (int r = 0; r < kExpandMaxK; ++r) {
      if (r < K) {
        const u32x2 p = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(ws, kExpandRowBase + lane * kExpandRowSlot + 8 * r, 0,
                                                        kWriteThrough));
        sc[r] = __uint_as_float(p.x);
        tk[r] = static_cast<int>(p.y);
      }
    }
  }
  int head = 0;  // slots of this leaf taken so far
  int out_leaf = 0, out_slot = 0, out_tok = 0;
  float out_score = 0.f;
#pragma unroll
  for (int r = 0; r < kExpandMaxK; ++r) {
    if (r < K) {
      const u64 hk = tk[0] >= 0 ? (static_cast<u64>(order_key(sc[0])) << 32) |
                                      static_cast<u64>(~static_cast<uint32_t>((lane << 8) | head))
                                : 0ull;
      const u64 w = wave_max_u64(hk);
      const uint32_t who = ~static_cast<uint32_t>(w);  // (leaf << 8) | slot
      const int src = static_cast<int>(who >> 8);
      const int win_tok = __builtin_amdgcn_readlane(tk[0], src);
      const float win_score = readlane_f32(sc[0], src);
      if (lane == r) {
        out_leaf = src;
        out_slot = static_cast<int>(who & 255u);
        out_tok = win_tok;
        out_score = win_score;
      }
      if (hk == w && w != 0) {
#pragma unroll
        for (int i = 0; i + 1 < kExpandMaxK; ++i) {
          sc[i] = sc[i + 1];
          tk[i] = tk[i + 1];
        }
        sc[kExpandMaxK - 1] = kNegInf;
        tk[kExpandMaxK - 1] = -1;
        ++head;
      }
    }
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
  if (dtype == TA_F32)
    hipLaunchKernelGGL(tree_expand_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  else if (dtype == TA_BF16)
    hipLaunchKernelGGL(tree_expand_kernel<__bf16>, grid, dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ta
