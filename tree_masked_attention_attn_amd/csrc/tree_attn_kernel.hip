// Tree-masked attention for gfx950 (CDNA4).
//
// What is computed (SwiftSpec, arXiv 2506.11309, Pith review page, "What
// carries the argument" and the referee summary): each tree token attends to
// the verified prefix, to its ancestors in the tree and to itself; the cache
// holds the prefix contiguously with the tree tokens right after it. The
// pages' kernel targets Hopper and hands partial results between thread
// blocks without explicit barriers; here the same idea is a per-row-block
// arrival count (device-scope atomics; the partial rows travel by
// device-scope stores and loads), after which each split merges its own
// slice of the block's rows, so the whole call is one launch with no grid
// barrier.
//
// Work decomposition (both kernels). A work unit is one workgroup: one KV
// head x one block of 128 of its query rows (64 in the bf16 sparse-block
// instance, which the plan picks for heads of at most 64 rows and where
// 128-row blocks would leave CUs idle; row r of a head is frontier
// node q_first + r / G, query head g*G + r % G, so a GQA group's rows share
// every K/V tile) x one contiguous range of 64-key stages (a "split" of
// [0, prefix_len + n_tree)). Splits spread the few KV heads over the 256 CUs;
// their partial (reference max, sum, unnormalised output) rows go to the
// workspace in fp32 and are merged in split order, so results are
// deterministic for a given shape.
//
// The fp32 kernel (the tiny fp32 shapes) stages K and V through registers
// into LDS with 4 waves of 32 rows. The bf16 kernel (below, with its own
// description) streams K and V by buffer-to-LDS DMA into rings of 64-key
// slots and runs 8 waves, two per SIMD. Both compute S^T = K Q^T with MFMA
// (keys = M, a wave's 32 rows = N, head_dim = K), so after the product every
// lane holds 16 scores of ONE row and the online softmax needs a single
// cross-lane exchange (lane ^ 32) per tile; O^T += V^T P^T keeps one row per
// lane as well, so the running-max rescale is a per-lane scalar.
//
// Ancestor mask: two 64-bit words per tree node (bit j = node j is the node
// itself or one of its ancestors; nodes 0..63 and 64..127), passed in the
// kernel arguments; only stages that reach past the prefix test them.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <type_traits>

#include "launch.h"

namespace ta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 32;     // keys per MFMA sub-tile (the M side of S^T = K Q^T)
constexpr int kSub = 2;       // sub-tiles per LDS stage
constexpr int kStage = kTile * kSub;
constexpr int kBlockRows = 128;
constexpr float kNegInf = -__builtin_huge_valf();

// x / d for 0 <= x < 2^17 and 1 <= d < 2^15, rcp as TreeAttnArgs documents:
// x * rcp / 2^32 exceeds x / d by less than 2^-15 < 1 / d, so its integer
// part is the quotient. Two instructions instead of a division sequence.
__device__ __forceinline__ int div_small(int x, int d, uint32_t rcp) {
  return d == 1 ? x : static_cast<int>(__umulhi(static_cast<uint32_t>(x), rcp));
}

// The work unit of workgroup b: its split, (KV head, row block) group and
// stage range. Consecutive workgroup ids go round-robin over the 8 XCDs, so
// each XCD gets a contiguous run of units: the row blocks and splits of one
// KV head then share that XCD's L2.
struct Unit {
  int u, split, grp, rb, g, t0, t1;
};

__device__ __forceinline__ Unit unit_of(const TreeAttnArgs& a, int b) {
  Unit w;
  w.u = (a.n_units % 8 == 0) ? (b % 8) * (a.n_units / 8) + b / 8 : b;
  w.grp = div_small(w.u, a.splits, a.splits_rcp);
  w.split = w.u - w.grp * a.splits;
  w.g = div_small(w.grp, a.row_blocks, a.row_blocks_rcp);
  w.rb = w.grp - w.g * a.row_blocks;
  w.t0 = w.split * a.split_stages + min(w.split, a.split_extra);
  w.t1 = w.t0 + a.split_stages + (w.split < a.split_extra ? 1 : 0);
  return w;
}

// Position of key `k` (0..31 within a sub-tile) inside a transposed V row in
// LDS. The PV MFMA reads, per lane half and k-slot, the keys that the S^T
// accumulator gave that lane; this permutation makes those keys contiguous so
// one wide LDS read fetches a whole operand.
template <typename T>
__device__ __forceinline__ int vpos(int k) {
  if constexpr (std::is_same_v<T, float>) {
    // f32 PV step t (0..15) of lane half h consumes key 8(t/4) + 4h + t%4.
    return ((k >> 2) & 1) * 16 + (k >> 3) * 4 + (k & 3);
  } else {
    // bf16 PV step ks (0..1), slot s (0..7) of half h: key 16ks + 8(s/4) + 4h + s%4.
    return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
  }
}

// One LDS stage holds kStage keys: K row-major [key][D] and V transposed
// [D][kStage] (each 32-key sub-tile permuted by vpos), both rows padded by 16
// bytes so the MFMA operand reads of 8 (or 16) consecutive lanes fall in
// distinct banks.
template <typename T, int D>
struct Layout {
  static constexpr int ES = sizeof(T);
  static constexpr int KSTR = D * ES + 16;
  static constexpr int VSTR = kStage * ES + 16;
  static constexpr int KBYTES = kStage * KSTR;
  static constexpr int BUF = KBYTES + D * VSTR;
  static constexpr int KCHUNKS = kStage * D * ES / 16;  // 16-B chunks of K per stage
  static constexpr int KREP = KCHUNKS / kThreads;
  static constexpr int VE = D / 16;                     // d values per key row per thread
  static constexpr int VW = VE * ES / 4;                // their 32-bit words (2, 4 or 8)
  static_assert(KCHUNKS % kThreads == 0, "K stage must split evenly over the threads");
};

template <typename T, int D>
struct Stage {
  uint4 kreg[Layout<T, D>::KREP];
  uint32_t vreg[4][Layout<T, D>::VW];  // 4 consecutive keys x VE d values
};

// Buffer resource over the K (or V) rows [k0, total_keys) of one head: loads
// at or beyond the end return 0 in hardware (raw-buffer range check), so the
// last stage needs no branches, and rows past total_keys are never read.
template <typename T, int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(const T* head, int k0, int total_keys) {
  const int left = total_keys - k0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(head + (size_t)k0 * D), 0,
                                           left > 0 ? left * D * (int)sizeof(T) : 0, 0x00020000);
}

template <int W>
__device__ __forceinline__ void buf_words(uint32_t (&dst)[W], __amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (W == 2) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    dst[0] = x[0]; dst[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
      dst[4 * i] = x[0]; dst[4 * i + 1] = x[1]; dst[4 * i + 2] = x[2]; dst[4 * i + 3] = x[3];
    }
  }
}

// Global -> registers for the stage starting at key `k0`.
// K: 16-B chunks in row order (a stage of K is contiguous in memory).
// V: thread t takes the 4 keys 4*(t%16) .. +3 and the VE head_dim values
// starting at (t/16)*VE, so that 16 consecutive lanes later write one whole
// transposed row segment (128 contiguous bytes for bf16): no bank conflicts.
template <typename T, int D>
__device__ __forceinline__ void load_stage(Stage<T, D>& st, const T* kh, const T* vh, int k0,
                                           int total_keys, int tid) {
  using L = Layout<T, D>;
  const __amdgpu_buffer_rsrc_t rk = stage_rsrc<T, D>(kh, k0, total_keys);
  const __amdgpu_buffer_rsrc_t rv = stage_rsrc<T, D>(vh, k0, total_keys);
#pragma unroll
  for (int r = 0; r < L::KREP; ++r) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, (tid + r * kThreads) * 16, 0, 0);
    st.kreg[r] = make_uint4(x[0], x[1], x[2], x[3]);
  }
  const int kg = tid & 15, dg = tid >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    buf_words<L::VW>(st.vreg[b], rv, ((kg * 4 + b) * D + dg * L::VE) * L::ES);
}

// Registers -> LDS stage: K row-major, V transposed with keys permuted.
template <typename T, int D>
__device__ __forceinline__ void store_stage(const Stage<T, D>& st, char* buf, int tid) {
  using L = Layout<T, D>;
  constexpr int CPR = D * L::ES / 16;
#pragma unroll
  for (int r = 0; r < L::KREP; ++r) {
    const int ci = tid + r * kThreads;
    *reinterpret_cast<uint4*>(buf + (ci / CPR) * L::KSTR + (ci % CPR) * 16) = st.kreg[r];
  }
  char* vt = buf + L::KBYTES;
  const int kg = tid & 15, dg = tid >> 4;
  // 4 consecutive keys stay contiguous under vpos; sub-tile kg/8 starts at key 32*(kg/8).
  const int col = ((kg >> 3) * kTile + vpos<T>((kg & 7) * 4)) * L::ES;
#pragma unroll
  for (int e = 0; e < L::VE; ++e) {
    char* dst = vt + (dg * L::VE + e) * L::VSTR + col;
    if constexpr (std::is_same_v<T, float>) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(st.vreg[0][e], st.vreg[1][e], st.vreg[2][e], st.vreg[3][e]);
    } else {
      // element e of each key row is 16-bit half (e % 2) of word e / 2; one
      // byte permute packs that half of two keys into one word
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      *reinterpret_cast<uint2*>(dst) =
          make_uint2(__builtin_amdgcn_perm(st.vreg[1][w], st.vreg[0][w], sel),
                     __builtin_amdgcn_perm(st.vreg[3][w], st.vreg[2][w], sel));
    }
  }
}

// Query fragments: the B operand of S^T = K Q^T for this lane's row.
template <typename T, int D>
struct QFrag {
  static constexpr int N = std::is_same_v<T, float> ? D / 2 : D / 16;
  using V = std::conditional_t<std::is_same_v<T, float>, float, bf16x8>;
  V f[N];
};

template <typename T, int D>
__device__ __forceinline__ void load_q(QFrag<T, D>& qf, const T* qrow, bool ok, int half) {
  if constexpr (std::is_same_v<T, float>) {
    // lane half h holds d in [h*D/2, (h+1)*D/2); MFMA step c uses d = h*D/2 + c.
#pragma unroll
    for (int c = 0; c < D / 2; c += 4) {
      f32x4 x = ok ? *reinterpret_cast<const f32x4*>(qrow + half * (D / 2) + c) : f32x4{0, 0, 0, 0};
      qf.f[c] = x[0]; qf.f[c + 1] = x[1]; qf.f[c + 2] = x[2]; qf.f[c + 3] = x[3];
    }
  } else {
    // MFMA step c covers d in [16c, 16c+16); lane half h holds d = 16c + 8h .. +7.
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      bf16x8 x = {};
      if (ok) x = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * half);
      qf.f[c] = x;
    }
  }
}

// S^T tile (32 keys x 32 rows) of one wave; lane (l32, half) gets the scores of
// row l32 for keys 8(j/4) + 4*half + j%4, j = 0..15.
template <typename T, int D>
__device__ __forceinline__ f32x16 qk_tile(const QFrag<T, D>& qf, const char* kbuf, int l32, int half) {
  using L = Layout<T, D>;
  f32x16 acc = {};
  const char* krow = kbuf + l32 * L::KSTR;  // kbuf: first key row of the sub-tile
  if constexpr (std::is_same_v<T, float>) {
#pragma unroll
    for (int c = 0; c < D / 2; c += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(krow + (half * (D / 2) + c) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf.f[c + e], acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (16 * c + 8 * half) * 2);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.f[c], acc, 0, 0, 0);
    }
  }
  return acc;
}

// O^T (D x 32 rows) += V^T P^T for one sub-tile; p[j] pairs with the key
// layout of qk_tile; vbuf points at the sub-tile's first column of V^T.
template <typename T, int D>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[D / 32], const float* p, const char* vbuf,
                                        int l32, int half) {
  using L = Layout<T, D>;
  if constexpr (std::is_same_v<T, float>) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const char* vrow = vbuf + (dt * 32 + l32) * L::VSTR + half * 16 * 4;
#pragma unroll
      for (int t = 0; t < 16; t += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(vrow + t * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], p[t + e], o[dt], 0, 0, 0);
      }
    }
  } else {
    bf16x8 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int s = 0; s < 8; ++s) pf[ks][s] = static_cast<__bf16>(p[8 * ks + s]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const char* vrow = vbuf + (dt * 32 + l32) * L::VSTR;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + (16 * ks + 8 * half) * 2);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[dt], 0, 0, 0);
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, f32x4 x) {
  if constexpr (std::is_same_v<T, float>) {
    *reinterpret_cast<f32x4*>(dst) = x;
  } else {
    bf16x4 y;
    y[0] = static_cast<__bf16>(x[0]); y[1] = static_cast<__bf16>(x[1]);
    y[2] = static_cast<__bf16>(x[2]); y[3] = static_cast<__bf16>(x[3]);
    *reinterpret_cast<bf16x4*>(dst) = y;
  }
}

// Split partials are stored in "lane order": for block row r (0..127) the
// float4 holding head_dim values 4c .. 4c+3 is element
//   ((r/32 * D/32 + c/8) * 4 + (c%8)/2) * 64 + (c%2) * 32 + r%32
// of the unit's [128 * D / 4] float4 array. That is exactly where lane
// (half, l32) of the wave owning 32-row tile r/32 holds those values in its
// O^T accumulator, so each partial store instruction writes 1 KB contiguously.
template <int D>
__device__ __forceinline__ int part_index(int r, int c) {
  return (((r >> 5) * (D / 32) + (c >> 3)) * 4 + ((c & 7) >> 1)) * 64 + (c & 1) * 32 + (r & 31);
}

// Split partials are written with device-scope stores (cache policy sc1): they
// go through this XCD's L2 to memory, so the release before the hand-off
// finds no dirty lines of theirs to write back. A plain store would leave
// them dirty, and every split's release would write back the XCD's whole
// backlog of partials, one split after another.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kWriteThrough = 16;

struct PartialSink {
  __amdgpu_buffer_rsrc_t o, ml;
};

template <int D>
__device__ __forceinline__ PartialSink partial_sink(const TreeAttnArgs& a, int u) {
  PartialSink k;
  const char* o = reinterpret_cast<const char*>(a.ws_o) + (size_t)u * kBlockRows * D * sizeof(float);
  k.o = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(o), 0, kBlockRows * D * (int)sizeof(float), 0x00020000);
  k.ml = __builtin_amdgcn_make_buffer_rsrc(a.ws_ml + (size_t)u * kBlockRows, 0, kBlockRows * 8, 0x00020000);
  return k;
}

// float4 number i of the unit's partial rows (lane order, see part_index)
__device__ __forceinline__ void put_partial(const PartialSink& k, int i, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), k.o, i * 16, 0, kWriteThrough);
}

// (reference max, sum) of block row r
__device__ __forceinline__ void put_ml(const PartialSink& k, int r, float m, float l) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, make_float2(m, l)), k.ml, r * 8, 0, kWriteThrough);
}

// Merge rows [r0, r1) of row block `grp` from all splits and write them to
// `out`: M is the running max of the splits' reference maxima, acc and L are
// rescaled by 2^(M_old - M), in split order (deterministic for a given shape).
// Device-scope loads (cache policy sc1), like the count that announced the
// partials: they do not return lines cached before the partials were
// written. A split index past the last one falls outside the buffer ranges
// and reads zeros without a memory access; it is ignored.
//
// One memory round trip per item: a thread loads every split's (max, sum)
// pair and partial float4 of its item before combining them.
//  * Up to 8 splits: an item is one (row, float4 column); consecutive threads
//    take consecutive rows, which are consecutive in the lane-ordered
//    partials (a wave's load touches a few cache lines, not one per lane
//    pair).
//  * 9 to 32 splits: an item is (row, column, group of 8 splits); the H = 2
//    or 4 groups of one (row, column) sit in adjacent lanes and are combined
//    with lane exchanges, so a slice of 128/S rows still takes one batch of
//    8 loads per thread instead of S/8 batches in a row.
template <typename T, int D, int NTH, int BR>  // BR: rows per row block
__device__ void merge_rows(const TreeAttnArgs& a, int grp, int g, int rb, int r0, int r1, int tid) {
  constexpr int block = BR;
  constexpr int C4 = D / 4;  // chunks of 4 values per row
  constexpr int MB = 8;      // splits per load batch
  const int S = a.splits;
  const size_t u0 = (size_t)grp * S;
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<f32x4*>(reinterpret_cast<const f32x4*>(a.ws_o) + u0 * kBlockRows * C4), 0,
      S * kBlockRows * C4 * (int)sizeof(f32x4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float2*>(a.ws_ml + u0 * kBlockRows), 0, S * kBlockRows * 8, 0x00020000);
  // Online combine of the splits s0 .. s0 + MB - 1 of (block row br, column c)
  // into (M, L, acc), after loading all of them.
  auto combine = [&](int br, int c, int s0, float& M, float& L, f32x4& acc) {
    const int pi = part_index<D>(br, c);
    float2 ml[MB];
    f32x4 o[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int sk = s0 + k;
      ml[k] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rm, (sk * kBlockRows + br) * 8, 0,
                                                                              kWriteThrough));
      o[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, (sk * kBlockRows * C4 + pi) * 16,
                                                                            0, kWriteThrough));
    }
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      // a split past the end, or one with no visible key for this row, adds nothing
      const bool ok = s0 + k < S && ml[k].x != kNegInf;
      const float Mn = ok ? fmaxf(M, ml[k].x) : M;
      const float sa = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float sb = ok ? __builtin_amdgcn_exp2f(ml[k].x - Mn) : 0.f;
      acc = acc * sa + o[k] * sb;
      L = L * sa + ml[k].y * sb;
      M = Mn;
    }
  };
  auto put = [&](int br, int c, float L, f32x4 acc) {
    const int hrow = rb * block + br;
    const int nd = div_small(hrow, a.group, a.group_rcp), hd = g * a.group + hrow - nd * a.group;
    store4<T>(static_cast<T*>(a.out) + ((size_t)nd * a.n_q_heads + hd) * D + 4 * c, acc * (1.f / L));
  };
  if (S <= MB) {
    constexpr int RPP = NTH / C4;  // rows per pass
    static_assert(RPP * C4 == NTH && (RPP & (RPP - 1)) == 0, "threads per pass");
    const int c = tid / RPP;
    for (int br = r0 + tid % RPP; br < r1; br += RPP) {
      if (rb * block + br >= a.rows_per_head) continue;
      float M = kNegInf, L = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      combine(br, c, 0, M, L, acc);
      put(br, c, L, acc);
    }
    return;
  }
  // H groups of 8 splits per (row, column), in lanes h = lane % H.
  const int H = S <= 2 * MB ? 2 : 4;
  const int h = tid & (H - 1);
  const int rows = r1 - r0;
  const int pairs = rows * C4;
  const int per_pass = NTH / H;
  const int passes = (pairs + per_pass - 1) / per_pass;  // uniform: every lane runs every pass
  for (int pass = 0; pass < passes; ++pass) {
    // every lane of a wave takes part in the exchanges below; an item past the
    // slice loads nothing
    const int p = pass * per_pass + tid / H;
    const bool live = p < pairs;
    const int br = r0 + (live ? p % rows : 0), c = live ? p / rows : 0;
    float M = kNegInf, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (live) combine(br, c, h * MB, M, L, acc);
    // combine the H groups, the lower group's terms first in every lane
#pragma unroll
    for (int step = 1; step < 4; step <<= 1) {
      if (step >= H) break;
      const float M2 = __shfl_xor(M, step), L2 = __shfl_xor(L, step);
      f32x4 a2;
#pragma unroll
      for (int i = 0; i < 4; ++i) a2[i] = __shfl_xor(acc[i], step);
      const float Mn = fmaxf(M, M2);
      const float sa = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float sb = M2 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M2 - Mn);
      const bool lower = (h & step) == 0;
      acc = lower ? acc * sa + a2 * sb : a2 * sb + acc * sa;
      L = lower ? L * sa + L2 * sb : L2 * sb + L * sa;
      M = Mn;
    }
    if (live && h == 0 && rb * block + br < a.rows_per_head) put(br, c, L, acc);
  }
}

// Cross-workgroup hand-off of one split, after its partial rows and (max,
// sum) pairs are in the workspace (no grid barrier, no second launch). Each
// row-block group has an arrival count and a word of give-up bits. One
// thread per workgroup:
//  * counts in with a wrapping increment: the count goes 0, 1, .., and back
//    to 0 at the last arrival, which leaves it ready for the next call.
//    Everything the split shares was written with device-scope stores
//    (through L2 to memory), so waiting for those stores to complete
//    (vmcnt 0) before a device-scope atomic publishes them; an agent-scope
//    release fence would also write back every dirty line of this XCD's L2,
//    which costs several microseconds and is not needed here;
//  * the others poll the count a bounded number of times until it has
//    wrapped (it is at most their own arrival number again). Readers then
//    load the partials with device-scope loads, which see memory as the
//    count does, so no acquire fence (which would invalidate the whole L2
//    of the XCD under the workgroups still streaming K and V) is needed;
//  * a split that saw the wrap merges its own row slice (slice j of the
//    block belongs to split j). One that stopped waiting sets its bit in the
//    give-up bits, waits for that atomic to complete and looks at the count
//    once more. The last arrival takes (and clears) the give-up bits after
//    its increment has been performed, merges its own slice while that
//    exchange is in flight, then every slice marked there. These atomics
//    are performed at one coherence point in the order each side completes
//    them: a bit set before the exchange is merged by the last arrival, one
//    set after it sees the wrap and is merged by its owner. A slice merged
//    twice is written twice with the same bytes, and a bit left set for a
//    later call only makes that call's last arrival merge a slice that is
//    already complete.
template <typename T, int D, int NTH, int BR>  // BR as for merge_rows
__device__ void split_handoff(const TreeAttnArgs& a, int* s_flags, int* s_mask, int grp, int g, int rb,
                              int split, int tid) {
  constexpr int block = BR;
  // Every wave waits for its own partial stores to complete before the
  // barrier (a workgroup barrier does not wait for global stores by itself),
  // so the whole workgroup's partials have been performed once thread 0
  // passes it.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* gw = reinterpret_cast<unsigned*>(a.ws_cnt) + (size_t)grp * 4;  // [0] arrivals, [2] give-up bits
  unsigned others = 0;
  if (tid == 0) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned old = __builtin_amdgcn_atomic_inc32(gw, a.splits - 1, __ATOMIC_RELAXED, "agent");
    int flag;
    if (old == (unsigned)a.splits - 1) {
      // the last arrival; the exchange result is first needed after its merge
      others = __hip_atomic_exchange(gw + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      flag = 2;
    } else {
      // Polls about 2048 cycles (~1 us) apart: shorter intervals measured
      // slower (up to 10% on the whole launch with 16 splits), the pollers'
      // device-scope loads of one address then crowding the memory traffic
      // that the last splits and the merges still need.
      bool all_in = false;
      for (int it = 0; !all_in && it < a.wait_polls; ++it) {
        __builtin_amdgcn_s_sleep(32);
        all_in = __hip_atomic_load(gw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= old;
      }
      if (!all_in) {
        __hip_atomic_fetch_or(gw + 2, 1u << split, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);  // the mark is performed before looking again
        all_in = __hip_atomic_load(gw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= old;
      }
      flag = all_in ? 1 : 0;
    }
    *s_flags = flag;
  }
  __syncthreads();
  const int flag = *s_flags;
  if (flag) merge_rows<T, D, NTH, BR>(a, grp, g, rb, div_small(split * block, a.splits, a.splits_rcp),
                                          div_small((split + 1) * block, a.splits, a.splits_rcp), tid);
  if (flag == 2) {
    if (tid == 0) *s_mask = static_cast<int>(others & ~(1u << split));
    __syncthreads();
    const unsigned marked = static_cast<unsigned>(*s_mask);
    for (int j = 0; j < a.splits; ++j)
      if ((marked >> j) & 1u)
        merge_rows<T, D, NTH, BR>(a, grp, g, rb, div_small(j * block, a.splits, a.splits_rcp),
                                      div_small((j + 1) * block, a.splits, a.splits_rcp), tid);
  }
}

// Scores more than 2^kSlack above the running reference trigger a rescale;
// smaller increases are absorbed (weights stay below 2^kSlack, exact after the
// final normalisation). This skips the O rescale on almost every tile.
constexpr float kSlack = 8.f;

// Waves per SIMD each instantiation is built for: two workgroups per CU,
// except fp32 with head_dim 128 whose LDS stages only fit one.
template <typename T, int D>
constexpr int kOccupancy = (std::is_same_v<T, float> && D == 128) ? 1 : 2;

template <typename T, int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kOccupancy<T, D>, kOccupancy<T, D>)))
void tree_attn_kernel(const TreeAttnArgs a) {
  using L = Layout<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::BUF];
  __shared__ int s_flags, s_taken;

  const Unit un = unit_of(a, blockIdx.x);
  const int u = un.u, split = un.split, grp = un.grp, rb = un.rb, g = un.g;
  const int t0 = un.t0, t1 = un.t1;  // in kStage-key stages

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int rloc = wave * 32 + l32;          // row within the block
  const int row = rb * kBlockRows + rloc;    // row within the KV head
  const bool row_ok = row < a.rows_per_head;
  const int node = row_ok ? div_small(row, a.group, a.group_rcp) : 0;  // query row (tree node q_first + node)
  const int head = g * a.group + (row_ok ? row - node * a.group : 0);
  const uint64_t anc = row_ok ? a.anc[a.q_first + node] : 0;        // tree nodes 0..63
  const uint64_t anc_hi = row_ok ? a.anc_hi[a.q_first + node] : 0;  // tree nodes 64..127

  const T* kh = static_cast<const T*>(a.k) + (size_t)g * a.kv_head_stride;
  const T* vh = static_cast<const T*>(a.v) + (size_t)g * a.kv_head_stride;

  QFrag<T, D> qf;
  load_q<T, D>(qf, static_cast<const T*>(a.q) + ((size_t)node * a.n_q_heads + head) * D, row_ok, half);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_ref = kNegInf, l_run = 0.f;

  Stage<T, D> st;
  load_stage<T, D>(st, kh, vh, t0 * kStage, a.total_keys, tid);
  store_stage<T, D>(st, smem, tid);
  // Every global load issued so far (q and the first stage) has landed: the
  // loop below then only ever waits for its own prefetch.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const float c = a.scale_log2;  // > 0, so the max of raw scores gives the max of scaled ones
  for (int stage = t0; stage < t1; ++stage) {
    char* cur = smem + ((stage - t0) & 1) * L::BUF;
    const bool more = stage + 1 < t1;
    if (more) load_stage<T, D>(st, kh, vh, (stage + 1) * kStage, a.total_keys, tid);

    float p[16 * kSub];
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const f32x16 sc = qk_tile<T, D>(qf, cur + sub * kTile * L::KSTR, l32, half);
#pragma unroll
      for (int j = 0; j < 16; ++j) p[16 * sub + j] = sc[j];
    }
    const int kb = stage * kStage;
    if (kb + kStage > a.prefix_len) {  // the stage reaches the tree (or past the end)
#pragma unroll
      for (int j = 0; j < 16 * kSub; ++j) {
        const int key = kb + kTile * (j >> 4) + 8 * ((j >> 2) & 3) + 4 * half + (j & 3);
        bool vis = key < a.prefix_len;
        if (!vis && key < a.total_keys) {
          const int t = key - a.prefix_len;
          vis = ((t < 64 ? anc >> t : anc_hi >> (t - 64)) & 1) != 0;
        }
        if (!vis) p[j] = kNegInf;
      }
    }
    float mx = p[0];
#pragma unroll
    for (int j = 1; j < 16 * kSub; ++j) mx = fmaxf(mx, p[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;  // both lane halves of a row agree
    const bool bump = mx > m_ref + kSlack;
    float alpha = 1.f;
    if (bump) {
      alpha = __builtin_amdgcn_exp2f(m_ref - mx);  // 0 on the first visible stage
      m_ref = mx;
    }
    const float nm = m_ref == kNegInf ? 0.f : -m_ref;  // nothing visible yet: weights are 0
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 16 * kSub; ++j) {
      p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(p[j], c, nm));
      psum += p[j];
    }
    l_run = l_run * alpha + psum;
    if (__ballot(bump)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
      pv_tile<T, D>(o, p + 16 * sub, cur + L::KBYTES + sub * kTile * L::ES, l32, half);

    if (more) store_stage<T, D>(st, smem + ((stage + 1 - t0) & 1) * L::BUF, tid);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  // Accumulator element j of o[dt] is d = 32 dt + 8 (j/4) + 4 half + j%4.
  if (a.splits == 1) {
    if (row_ok) {
      T* orow = static_cast<T*>(a.out) + ((size_t)node * a.n_q_heads + head) * D;
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          f32x4 x = {o[dt][4 * jq], o[dt][4 * jq + 1], o[dt][4 * jq + 2], o[dt][4 * jq + 3]};
          store4<T>(orow + 32 * dt + 8 * jq + 4 * half, x * inv);
        }
    }
    return;
  }

  // Publish this split's rows (reference max, sum, unnormalised output), then hand off.
  {
    const PartialSink sink = partial_sink<D>(a, u);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        put_partial(sink, ((wave * (D / 32) + dt) * 4 + jq) * 64 + lane,
                    f32x4{o[dt][4 * jq], o[dt][4 * jq + 1], o[dt][4 * jq + 2], o[dt][4 * jq + 3]});
    if (half == 0) put_ml(sink, rloc, m_ref, l_tot);
  }
  split_handoff<T, D, kThreads, kBlockRows>(a, &s_flags, &s_taken, grp, g, rb, split, tid);
}

// ============================================================================
// bf16 kernel. Same maths and hand-off as above, built for CDNA4's balance of
// MFMA, VALU and LDS:
//  * 8 waves, two per SIMD: 4 row groups (one 32-row MFMA N tile each) x 2
//    key halves. Wave w takes row group w % 4 and, of every 64-key stage,
//    the 32-key half w / 4; waves w and w + 4 share a SIMD. The two halves'
//    partial rows are merged through LDS at the end, each wave of the pair
//    combining and storing half of the head_dim columns.
//  * The two waves of a SIMD run each iteration in opposite orders: one
//    issues its MFMAs (PV of stage s - 1, QK of stage s + 1) and then the
//    softmax of stage s, the other the softmax first. Between the workgroup
//    barriers that start each iteration the matrix core works for one wave
//    while the VALU works for the other.
//  * A block of at most 64 query rows (every block of the sparse instance,
//    whose blocks are 64 rows, and the last block of a head in the dense
//    one) pairs each wave of real rows with a padding wave that only loads,
//    so every real wave has its SIMD to itself; its softmax is then free to
//    interleave with its MFMAs.
//  * NT (32-row tiles per wave) is 1. NT = 2, one wave per SIMD holding two
//    row tiles so that each K or V fragment feeds two MFMAs, was measured as
//    a variant of this kernel (its DMA split over four waves): same outputs,
//    slower. The register state and the iteration keep the parameter; the
//    DMA code here assumes eight waves.
//  * K and V reach LDS by buffer-to-LDS DMA (no staging registers, no VALU)
//    into two rings of four 64-key slots; each slot is refilled three
//    iterations before it is read. Q and the ancestor table are staged the
//    same way, so the compiler sees no vector-memory loads and every wait on
//    memory is an explicit vmcnt. Rows are stored as-is with their 16-byte
//    chunks XOR-swizzled by row, so the K operand reads (ds_read_b128) and
//    the transposed V reads (ds_read_b64_tr_b16, which hand each lane 4 keys
//    of one head_dim column) are free of bank conflicts. Keys past
//    prefix_len + n_tree fall outside the buffer range and arrive as zeros.
// ============================================================================
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// NT: 32-row MFMA tiles per wave. A workgroup's waves cover 128 rows (of
// which a 64-row block uses two tiles) and both 32-key halves of each stage:
// 8 / NT waves (NT = 1: two waves per SIMD; NT = 2: one wave per SIMD, each
// K or V fragment feeding two MFMAs).
#ifndef TA_BF16_NT
#define TA_BF16_NT 1
#endif
template <int NT>
constexpr int kBfWaves = 8 / NT;
template <int NT>
constexpr int kBfThreads = 64 * kBfWaves<NT>;
constexpr int kRing = 4;  // slots per ring (K and V each)

// LDS layout. LDS has 64 banks of 4 bytes: 16 sixteen-byte bank groups per
// 256 bytes, served to 16 lanes of a ds_read_b128 or 32 lanes of a
// ds_read_b64_tr_b16 at a time. K, Q and V rows are stored unpadded, with
// their 16-byte chunks permuted by XOR within the row:
//  * K (and Q): chunk c of row r sits at c ^ bf_ksw(r), bf_ksw(r) = r mod 16
//    (D = 128) or (r / 2) mod 8 (D = 64). A K fragment read has 16 lanes on
//    16 consecutive rows at one chunk: their bank groups are all distinct.
//  * V: chunk c of row r sits at c ^ 4 bf_vsw(r), bf_vsw(r) = r mod 4
//    (D = 128) or (r / 2) mod 2 (D = 64). A transposed read has 32 lanes on
//    rows r0 + e (e < 4, r0 a multiple of 4) and chunks 4t + j (j < 4):
//    their bank groups are all distinct.
// A 64-key slot is D/8 DMA instructions of 64 lanes x 16 bytes, KOPS per
// wave. Each instruction covers whole rows, and instruction o of a wave
// starts o * 8 KiB after its first; both swizzles repeat within that
// distance, so one per-lane source offset serves all of a wave's
// instructions (the rest is a wave-uniform addition).
template <int D>
struct BfGeo {
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int ROWB = D * 2;                  // bytes per row, in HBM and in LDS
  static constexpr int SLOT = 64 * ROWB;              // one 64-key K or V stage
  static constexpr int KOPS = CPR / 8;                // DMA instructions per wave per slot
  static constexpr int VRING = kRing * SLOT;          // the V ring follows the K ring
  static constexpr int QSTAGE0 = 3 * SLOT;            // Q rows 0-63 wait in K slot 3
  static constexpr int ANC = 2 * kRing * SLOT;        // ancestor words: [2][kMaxTree] x u64
  static constexpr int QSTAGE1 = ANC + 2048;          // Q rows 64-127
  static constexpr int LDS = QSTAGE1 + SLOT;
  static_assert(kBlockRows == 128 && CPR % 8 == 0, "layout");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int D>
__device__ __forceinline__ int bf_ksw(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int bf_vsw(int r) {
  return D == 128 ? (r & 3) : ((r >> 1) & 1);
}

// vmcnt(n) with every other counter left alone (gfx9 encoding).
#define TA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// vmcnt(x) for a wave-uniform x, rounded down to an even number (waiting
// for more than needed is always safe).
__device__ __forceinline__ void wait_vm_atmost(int x) {
  if (x >= 24) TA_WAIT_VM(24);
  else if (x >= 22) TA_WAIT_VM(22);
  else if (x >= 20) TA_WAIT_VM(20);
  else if (x >= 18) TA_WAIT_VM(18);
  else if (x >= 16) TA_WAIT_VM(16);
  else if (x >= 14) TA_WAIT_VM(14);
  else if (x >= 12) TA_WAIT_VM(12);
  else if (x >= 10) TA_WAIT_VM(10);
  else if (x >= 8) TA_WAIT_VM(8);
  else if (x >= 6) TA_WAIT_VM(6);
  else if (x >= 4) TA_WAIT_VM(4);
  else if (x >= 2) TA_WAIT_VM(2);
  else TA_WAIT_VM(0);
}

__device__ __forceinline__ void bf_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw-buffer resource (gfx9 layout) over `bytes` bytes at `base`, held in SGPRs.
__device__ __forceinline__ i32x4 bf_rsrc(const void* base, int bytes) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(p & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(p >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);                      // range: zero beyond
  r[3] = 0x00020000;
  return r;
}

// One 16-byte-per-lane buffer-to-LDS DMA: lane i's 16 bytes from byte `voff`
// of the resource land at LDS address lds + 16 i. Issued through asm so the
// compiler neither sees an LDS write nor inserts waits for it; every wait on
// these loads is explicit (TA_WAIT_VM), and the barriers order them against
// the LDS reads.
__device__ __forceinline__ void bf_dma16(i32x4 rsrc, unsigned lds, int voff) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(rsrc)
               : "memory", "m0");
}

// ... with a wave-uniform byte offset `add` on every lane's source. It goes
// into the per-lane offset, not the scalar one, so that the raw-buffer range
// check (which covers only the per-lane and instruction offsets) sees it.
__device__ __forceinline__ void bf_dma16(i32x4 rsrc, unsigned lds, int voff, int add) {
  bf_dma16(rsrc, lds, voff + add);
}

// Per-lane source offset (within a 64-key stage) of a wave's first DMA
// instruction into a K slot (KEY) or a V slot: LDS position
// p = 64 wave + lane = row * D/8 + physical chunk holds chunk
// (physical chunk) ^ swizzle(row) of the row. The wave's instruction o reads
// o * 8 KiB further on (the swizzles of row and row + 32 o agree).
template <int D, bool KEY>
__device__ __forceinline__ int bf_dma_offset(int wave, int lane) {
  using G = BfGeo<D>;
  const int p = wave * 64 + lane;
  const int row = p / G::CPR, pc = p % G::CPR;
  const int ch = KEY ? pc ^ bf_ksw<D>(row) : pc ^ (4 * bf_vsw<D>(row));
  return row * G::ROWB + ch * 16;
}

// DMA keys [k0, k0 + 64) of one head's K (or V) into a slot; `off` from
// bf_dma_offset.
template <int D, int NW>
__device__ __forceinline__ void bf_dma_slot(unsigned slot, const __bf16* head, int k0, int total_keys, int off,
                                            int wave) {
  using G = BfGeo<D>;
  const i32x4 r = bf_rsrc(head + (size_t)k0 * D, max(total_keys - k0, 0) * G::ROWB);
#pragma unroll
  for (int o = 0; o < G::KOPS; ++o) bf_dma16(r, slot + (o * NW + wave) * 1024, off, o * NW * 1024);
}

// DMA 128 query rows from the block's first (K layout; rows 0-63 into K
// slot 3, rows 64-127 into their own area; rows past the head's rows read as
// zeros; in a 64-row block rows 64-127 are the next block's and go unused)
// and, from the kernel arguments, the ancestor table.
template <int D, int NW>
__device__ __forceinline__ void bf_dma_q_anc(unsigned lds, const TreeAttnArgs& a, int g, int rb, int brows,
                                             int wave, int lane) {
  using G = BfGeo<D>;
  const int qbytes = (a.n_tree - a.q_first) * a.n_q_heads * G::ROWB;
  const i32x4 r = bf_rsrc(a.q, qbytes);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int o = 0; o < G::KOPS; ++o) {
      const int op = o * NW + wave;
      const int p = op * 64 + lane;
      const int row = p / G::CPR, ch = (p % G::CPR) ^ bf_ksw<D>(row);
      const int hr = rb * brows + 64 * h + row;  // h = 1 of a 64-row block: the next block, unused
      int off = qbytes;  // out of range: zeros
      if (hr < a.rows_per_head) {
        const int nd = div_small(hr, a.group, a.group_rcp);
        off = (nd * a.n_q_heads + g * a.group + hr - nd * a.group) * G::ROWB + ch * 16;
      }
      bf_dma16(r, lds + (h ? G::QSTAGE1 : G::QSTAGE0) + op * 1024, off);
    }
  if (wave == 0) {
    // The arguments block sits at the start of the kernarg segment; its two
    // 1 KB ancestor tables (words of nodes 0..63, then of nodes 64..127) are
    // adjacent and land in LDS as [2][kMaxTree] words.
    static_assert(offsetof(TreeAttnArgs, anc_hi) == offsetof(TreeAttnArgs, anc) + kMaxTree * 8, "tables");
    const char* args = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    const i32x4 ra = bf_rsrc(args + offsetof(TreeAttnArgs, anc), 2 * kMaxTree * 8);
    bf_dma16(ra, lds + G::ANC, lane * 16);
    bf_dma16(ra, lds + G::ANC + kMaxTree * 8, lane * 16 + kMaxTree * 8);
  }
}

// Max of 16 scores with the NaN-propagating maximum (v_maximum3_f32 on
// gfx950): fmaxf's NaN rules would cost an extra canonicalising instruction
// per input. Scores are finite or -inf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

template <typename R>  // float[16] or f32x16
__device__ __forceinline__ float max16(const R& p) {
  const float a = vmax(vmax(p[0], p[1]), p[2]);
  const float b = vmax(vmax(p[3], p[4]), p[5]);
  const float c = vmax(vmax(p[6], p[7]), p[8]);
  const float d = vmax(vmax(p[9], p[10]), p[11]);
  const float e = vmax(vmax(p[12], p[13]), p[14]);
  return vmax(vmax(vmax(a, b), c), vmax(vmax(d, e), p[15]));
}

template <typename R>  // float[16] or f32x16
__device__ __forceinline__ float sum16(const R& p) {  // fixed pairwise order
  float a0 = (p[0] + p[1]) + (p[2] + p[3]);
  float a1 = (p[4] + p[5]) + (p[6] + p[7]);
  float a2 = (p[8] + p[9]) + (p[10] + p[11]);
  float a3 = (p[12] + p[13]) + (p[14] + p[15]);
  return (a0 + a1) + (a2 + a3);
}

// v_permlane32_swap: a = [a_lo, b_lo], b = [a_hi, b_hi] (lo/hi: lanes 0-31 /
// 32-63). Written as asm because the compiler builtin returns its first
// result for both halves; the s_nop covers the VALU-write hazard on the
// operands.
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

template <int D, int NT>
struct BfWave {
  bf16x8 qf[NT][D / 16];  // Q fragments of the wave's row tiles
  f32x16 o[NT][D / 32];   // O^T accumulators
  float m_ref[NT], l_run[NT];
  float alpha[NT];        // rescale of O owed by the last softmax (applied before the next PV)
  bool pend;              // some row of the wave owes one
  unsigned anc_at[NT];    // LDS address of the row's first ancestor word (the second is kMaxTree words on)
};

// Settle the rescale the last softmax owes O. Kept a real branch (the asm
// stops the compiler from speculating 128 multiplies): references move
// rarely, by design of the lazy maximum.
template <int D, int NT>
__device__ __forceinline__ void bf_rescale(BfWave<D, NT>& w) {
  if (w.pend) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) w.o[nt][dt] *= w.alpha[nt];
  }
}

// K fragments of the wave's 32-key half: K rows 32 kh + l32, chunk 2 cc + half
// (also the Q fragments, from a Q staging area). Under the swizzle the
// chunk sits at 2 (cc ^ s1) + (half ^ s0), s = bf_ksw(row): fragment cc of
// every lane is at (its fragment-0 address) ^ 32 cc.
template <int D>
__device__ __forceinline__ void bf_read_k(bf16x8 (&kf)[D / 16], unsigned slot, int kh, int lane) {
  using G = BfGeo<D>;
  const int row = 32 * kh + (lane & 31), sw = bf_ksw<D>(row);
  const unsigned base = slot + row * G::ROWB + 32 * (sw >> 1) + 16 * ((lane >> 5) ^ (sw & 1));
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc)
    kf[cc] = *(__attribute__((address_space(3))) const bf16x8*)(unsigned long)(base ^ (32u * cc));
}

// V^T fragments (A operand of O^T += V^T P^T, 32 head_dim rows x 16 keys) of
// the wave's half, from two transposed reads each: lane (g = lane/16,
// j = lane%16) of a 16-lane group points at V[key e = j/4][head_dim
// 16 (g%2) + 4 (j%4) ..] and receives, for head_dim 16 (g%2) + j, the 4 keys
// the group pointed at. The rows a read touches share bf_vsw, and the
// swizzle only moves 64-byte column blocks, so head_dim block dt of every
// lane is at (its block-0 address) ^ 64 dt; rows further down are
// compile-time offsets.
template <int D>
__device__ __forceinline__ void bf_read_v(bf16x8 (&vf)[2][D / 32], unsigned slot, int kh, int lane) {
  using G = BfGeo<D>;
  constexpr int RS = G::ROWB;  // row stride, bytes
  const int half = lane >> 5, e = (lane & 15) >> 2, q = lane & 3, g1 = (lane >> 4) & 1;
  const int row = 32 * kh + 4 * half + e;
  const unsigned base = slot + row * RS + 64 * bf_vsw<D>(row) + (2 * g1 + (q >> 1)) * 16 + (q & 1) * 8;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const unsigned at = base ^ (64u * dt);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4v*)(unsigned long)(at + 16 * ks * RS));
      const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4v*)(unsigned long)(at + (16 * ks + 8) * RS));
      vf[ks][dt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// S^T = K Q^T for the wave's row tiles (keys = M, rows = N, head_dim = K): after
// the product lane (l32, half) holds, for row l32 of the tile, the scores of
// keys 8 (j/4) + 4 half + j%4 of the half, j = 0..15.
template <int D, int NT>
__device__ __forceinline__ void bf_qk(f32x16 (&s)[NT], const bf16x8 (&kf)[D / 16], const BfWave<D, NT>& w) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) s[nt] = f32x16{};
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cc], w.qf[nt][cc], s[nt], 0, 0, 0);
}

// O^T += V^T P^T for the wave's row tiles.
template <int D, int NT>
__device__ __forceinline__ void bf_pv(BfWave<D, NT>& w, const bf16x8 (&vf)[2][D / 32], const bf16x8 (&p)[NT][2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        w.o[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks][dt], p[nt][ks], w.o[nt][dt], 0, 0, 0);
}

// Visibility of the 32 keys kb .. kb + 31 for a row whose ancestor-or-self
// set is (hi:lo), tree nodes 0..127: bit i set iff key kb + i is a prefix key
// or one of the row's tree nodes (the set has no bits past n_tree, so keys
// past the end are hidden).
__device__ __forceinline__ uint32_t visible32(uint64_t lo, uint64_t hi, int kb, int prefix_len) {
  const int d = kb - prefix_len;  // key kb is tree node d when d >= 0
  const unsigned __int128 set = (static_cast<unsigned __int128>(hi) << 64) | lo;
  uint32_t tree;
  if (d >= 0) tree = d < 2 * 64 ? static_cast<uint32_t>(set >> d) : 0u;
  else tree = d > -32 ? static_cast<uint32_t>(lo << (-d)) : 0u;
  const uint32_t pre = d <= -32 ? ~0u : (d >= 0 ? 0u : ((1u << (-d)) - 1u));
  return pre | tree;
}

// In the scores x of one stage (keys kb .. kb + 31 of this half), set tree
// keys that are not ancestors of the row (and keys past the end) to -inf.
// The mask is a uniform branch taken only by stages that reach the tree.
template <int D, int NT, typename X>  // X: float[NT][16] or f32x16[NT]
__device__ __forceinline__ void bf_mask(const BfWave<D, NT>& w, X& x, int kb, int half, const TreeAttnArgs& a) {
  if (kb + 32 > a.prefix_len) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const auto* set = (__attribute__((address_space(3))) const uint64_t*)(unsigned long)w.anc_at[nt];
      const uint32_t vis = visible32(set[0], set[kMaxTree], kb, a.prefix_len) >> (4 * half);  // then constant bit tests
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (!((vis >> (8 * (j >> 2) + (j & 3))) & 1u)) x[nt][j] = kNegInf;
    }
  }
}

// How softmax forms the row sum, measured per head dim (A/B on MI355X):
// for 128, from the bf16 weights with v_dot2c, a serial chain left free to
// overlap the MFMAs of the softmax-first wave (3% faster at 70B shapes);
// for 64, whose MFMA block is half as long, as a pairwise fp32 tree of the
// unrounded weights, finished before the MFMAs (the chain costs 2% there).
template <int D>
constexpr bool kBfDotSum = D == 128;

// Online softmax of one stage: scores x (masked) -> bf16 weights pn. The
// reference max is raised lazily (only when a score exceeds it by more than
// 2^kSlack); the factors alpha that rescale O then wait in the wave state
// until the next PV.
template <int D, int NT, typename X>  // X: float[NT][16] or f32x16[NT]
__device__ __forceinline__ void bf_softmax(BfWave<D, NT>& w, X& x, bf16x8 (&pn)[NT][2], float c) {
  float mx[NT], nm[NT];
  // Row maxima over this lane's 16 keys, then over both lane halves.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) mx[nt] = max16(x[nt]);
  if constexpr (NT == 2) {
    swap32(mx[0], mx[1]);
    float mt = vmax(mx[0], mx[1]), mt2 = mt;  // lanes 0-31: tile 0's max; 32-63: tile 1's
    swap32(mt, mt2);                          // mt: tile 0's max everywhere, mt2: tile 1's
    mx[0] = mt;
    mx[1] = mt2;
  } else {
    float lo = mx[0], hi = mx[0];
    swap32(lo, hi);  // lo: the low half's max everywhere, hi: the high half's
    mx[0] = vmax(lo, hi);
  }
  bool bump_any = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float m = mx[nt] * c;
    const bool bump = m > w.m_ref[nt] + kSlack;
    const float al = __builtin_amdgcn_exp2f(w.m_ref[nt] - m);  // 0 on the first visible keys
    w.alpha[nt] = bump ? al : 1.f;
    w.m_ref[nt] = bump ? m : w.m_ref[nt];
    bump_any |= bump;
    nm[nt] = w.m_ref[nt] == kNegInf ? 0.f : -w.m_ref[nt];
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[nt][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nt][j], c, nm[nt]));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < 8; ++q) pn[nt][ks][q] = static_cast<__bf16>(x[nt][8 * ks + q]);
    if constexpr (kBfDotSum<D>) {
      // the bf16 weights that PV multiplies, two per instruction
      // (v_dot2c_f32_bf16 against 1.0, fp32 accumulation)
      float l = w.l_run[nt] * w.alpha[nt];
      const bf16x2v one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 v = pn[nt][ks];
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, l, false);
      }
      w.l_run[nt] = l;
    } else {
      w.l_run[nt] = w.l_run[nt] * w.alpha[nt] + sum16(x[nt]);
    }
  }
  w.pend = __ballot(bump_any) != 0;
}

// The MFMAs of one iteration, PV first (its operands are in registers since
// the previous iteration), then QK into sn, with the wave's NOPS DMA
// instructions spread evenly between them: a stall on a busy load path then
// costs nothing while the MFMA pipe is full.
template <int D, int NT, bool QK, bool PV, int NOPS, typename Dma, bool FENCE = true>
__device__ __forceinline__ void bf_mfma_block(BfWave<D, NT>& w, f32x16 (&sn)[NT], const bf16x8 (&kf)[D / 16],
                                              const bf16x8 (&vf)[2][D / 32], const bf16x8 (&pp)[NT][2], Dma&& dma) {
  constexpr int NPV = PV ? 2 * (D / 32) * NT : 0;  // k-steps x head_dim tiles x row tiles
  constexpr int NQK = QK ? (D / 16) * NT : 0;      // k-steps x row tiles
  constexpr int NM = NPV + NQK;
  if constexpr (QK) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sn[nt] = f32x16{};
  }
  static_assert(NOPS <= NM, "one DMA instruction per MFMA at most");
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i < NPV) {
      const int ks = i / ((D / 32) * NT), dt = (i / NT) % (D / 32), nt = i % NT;
      w.o[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks][dt], pp[nt][ks], w.o[nt][dt], 0, 0, 0);
    } else {
      const int k = i - NPV, cc = k / NT, nt = k % NT;
      sn[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cc], w.qf[nt][cc], sn[nt], 0, 0, 0);
    }
    if constexpr (NOPS > 0) {
      if ((i * NOPS) % NM == 0 && i * NOPS / NM < NOPS) {  // spread evenly, kept in place
        if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
        dma(i * NOPS / NM);
        if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// A uniform true that the compiler cannot see through. Code under it keeps
// a basic block of its own, so instruction selection cannot interleave it
// with the code around it.
__device__ __forceinline__ bool bf_opaque_true() {
  int one;
  asm volatile("s_mov_b32 %0, 1" : "=s"(one));
  return one != 0;
}

// Values pinned here are final at this point of the instruction stream (the
// compiler can neither sink their computation below nor hoist later uses
// above). Empty asm; the operands only carry the dependence.
template <typename T>
__device__ __forceinline__ void bf_pin(T& x) {
  static_assert(sizeof(T) == 4, "one register");
  asm volatile("" : "+v"(x));
}
template <int NT>
__device__ __forceinline__ void bf_pin_scores(float (&x)[NT][16]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 16; ++j) bf_pin(x[nt][j]);
}
template <int NT>
__device__ __forceinline__ void bf_pin_weights(bf16x8 (&p)[NT][2]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 u = __builtin_bit_cast(u32x4, p[nt][ks]);
      asm volatile("" : "+v"(u));
      p[nt][ks] = __builtin_bit_cast(bf16x8, u);
    }
}

// One pipeline iteration on stage j (QK, PV, VN select the parts that exist):
//  * settle the rescale softmax(j - 1) owes O;
//  * PV(j - 1) from the V fragments `vf` and the weights `pp`, and QK(j + 1)
//    from the K slot `knext` (its fragments are read first) -> new scores;
//  * softmax(j) of the scores `sc` -> the weights for PV(j);
//  * read V(j) from `vcur` into `vf` for the next iteration's PV.
// The two waves that share a SIMD run these in opposite orders: one issues
// its MFMAs first and then the softmax, the other the softmax first. Between
// the workgroup barriers that start each iteration, the matrix core then
// works for one wave while the vector ALU works for the other, instead of
// both waves contending for the same unit at the same time.
template <bool MFMA_FIRST, int D, int NT, bool QK, bool PV, bool VN, int NOPS, typename Dma, bool FREE = false>
__device__ __forceinline__ void bf_iter(BfWave<D, NT>& w, f32x16 (&sc)[NT], bf16x8 (&pp)[NT][2],
                                        bf16x8 (&vf)[2][D / 32], unsigned knext, unsigned vcur, int kb,
                                        int kh, int lane, const TreeAttnArgs& a, Dma&& dma) {
  bf16x8 kf[D / 16];
  float x[NT][16];
  if constexpr (PV) bf_rescale<D, NT>(w);
  if constexpr (FREE) {
    // A wave alone on its SIMD: no partner to hand the units to, so the
    // softmax is free to interleave with the MFMAs (mask first: its branch
    // would split the block).
    bf_mask<D, NT>(w, sc, kb, lane >> 5, a);
    if constexpr (QK) bf_read_k<D>(kf, knext, kh, lane);
    f32x16 sn[NT];
    bf16x8 pn[NT][2];
    bf_mfma_block<D, NT, QK, PV, NOPS, Dma, false>(w, sn, kf, vf, pp, dma);
    bf_softmax<D, NT>(w, sc, pn, a.scale_log2);
    if constexpr (VN) bf_read_v<D>(vf, vcur, kh, lane);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      pp[nt][0] = pn[nt][0];
      pp[nt][1] = pn[nt][1];
      if constexpr (QK) sc[nt] = sn[nt];
    }
  } else if constexpr (MFMA_FIRST) {
    // K fragments first: the PV MFMAs cover their latency
    if constexpr (QK) bf_read_k<D>(kf, knext, kh, lane);
    f32x16 sn[NT];
    if (bf_opaque_true()) bf_mfma_block<D, NT, QK, PV, NOPS>(w, sn, kf, vf, pp, dma);
    if constexpr (VN) bf_read_v<D>(vf, vcur, kh, lane);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) x[nt][j] = sc[nt][j];
    bf_pin_scores<NT>(x);  // the softmax starts only here
    bf_mask<D, NT>(w, x, kb, lane >> 5, a);
    bf_softmax<D, NT>(w, x, pp, a.scale_log2);
    if constexpr (QK) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sc[nt] = sn[nt];
    }
  } else {
    bf16x8 pn[NT][2];
    // in place: the scores are dead once the weights exist, and QK below
    // writes the next stage's into the same registers
    bf_mask<D, NT>(w, sc, kb, lane >> 5, a);
    bf_softmax<D, NT>(w, sc, pn, a.scale_log2);
    bf_pin_weights<NT>(pn);  // the softmax is done before the MFMAs
    if constexpr (!kBfDotSum<D>) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bf_pin(w.l_run[nt]);
    }
    // K fragments only now (not live through the softmax); the PV MFMAs
    // cover their latency
    if constexpr (QK) bf_read_k<D>(kf, knext, kh, lane);
    if (bf_opaque_true()) bf_mfma_block<D, NT, QK, PV, NOPS>(w, sc, kf, vf, pp, dma);
    if constexpr (VN) bf_read_v<D>(vf, vcur, kh, lane);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      pp[nt][0] = pn[nt][0];
      pp[nt][1] = pn[nt][1];
    }
  }
}

template <int D, int NT, bool SPARSE>
__global__ __launch_bounds__(kBfThreads<NT>)
__attribute__((amdgpu_waves_per_eu(kBfWaves<NT> / 4, kBfWaves<NT> / 4)))  // waves per SIMD
void tree_attn_bf16_kernel(const TreeAttnArgs a) {
  using G = BfGeo<D>;
  __shared__ __attribute__((aligned(1024))) char lds[G::LDS];
  __shared__ int s_flags, s_taken;
  __shared__ int s_pair[4];  // waves seen per SIMD

  const Unit un = unit_of(a, blockIdx.x);
  const int u = un.u, split = un.split, grp = un.grp, rb = un.rb, g = un.g;
  const int t0 = un.t0, t1 = un.t1;  // in 64-key stages
  const int n = t1 - t0;             // >= 1

  // wave is uniform: readfirstlane lets the compiler keep it (and all that
  // derives from it) in scalar registers, with scalar branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  constexpr int NW = kBfWaves<NT>, RW = NW / 2;  // waves, row groups
  // Row group and key half of the wave. Waves w and w + 4 share a SIMD. In a
  // block of at most 64 query rows (half or more of it padding), each SIMD
  // pairs a wave of real rows with a padding wave, and padding waves only
  // load: every real wave then has its SIMD to itself. Otherwise a SIMD
  // holds the two key halves of one row group.
  // rows per row block: 64 in the sparse-block instance, 128 otherwise
  constexpr int brows = SPARSE ? kBlockRows / 2 : kBlockRows;
  const int block_rows = min(a.rows_per_head - rb * brows, brows);
  const bool sparse = SPARSE || block_rows <= 64;
  const int rg = sparse ? 2 * (wave >> 2) + ((wave & 3) >> 1) : wave % RW;
  const int kh = sparse ? wave & 1 : wave / RW;
  // no row of this wave's tiles is a query row: it issues its share of the
  // loads and takes part in every barrier, nothing else
  const bool idle = sparse && 32 * NT * rg >= block_rows;
  const __bf16* kh_ptr = static_cast<const __bf16*>(a.k) + (size_t)g * a.kv_head_stride;
  const __bf16* vh_ptr = static_cast<const __bf16*>(a.v) + (size_t)g * a.kv_head_stride;
  // LDS byte addresses (the space the DMA and the fragment reads take)
  const unsigned lds0 = static_cast<unsigned>(
      reinterpret_cast<unsigned long>((__attribute__((address_space(3))) char*)lds));
  auto kslot = [&](int j) { return lds0 + (j & (kRing - 1)) * G::SLOT; };
  auto vslot = [&](int j) { return lds0 + G::VRING + (j & (kRing - 1)) * G::SLOT; };
  static_assert(NW == 8, "a slot is D/8 instructions, D/64 per wave");
  const int koff = bf_dma_offset<D, true>(wave, lane);
  const int voff = bf_dma_offset<D, false>(wave, lane);
  auto dma_k = [&](int j) {
    bf_dma_slot<D, NW>(kslot(j), kh_ptr, (t0 + j) * 64, a.total_keys, koff, wave);
  };
  auto dma_v = [&](int j) {
    bf_dma_slot<D, NW>(vslot(j), vh_ptr, (t0 + j) * 64, a.total_keys, voff, wave);
  };

  if (!SPARSE && tid < 4) s_pair[tid] = 0;

  // DMA issue order (j = stage index within the split): Q and ancestors, K0,
  // K1, K2, V0, V1, V2; iteration 0 issues K3, K4, V3 (over the Q staging
  // areas, after Q has been read); iteration j >= 1 issues K(j+4), V(j+3).
  // Iteration j needs K(j+1) and V(j); each wait counts the DMA instructions
  // issued after the newest of those, which may stay in flight.
  // The first burst carries only what the first two iterations read first
  // (Q, the ancestors, K0, K1, V0); K2, V1 and V2 follow once Q and K0 have
  // landed, so that those do not queue behind the whole chip's later stages.
  bf_dma_q_anc<D, NW>(lds0, a, g, rb, brows, wave, lane);
  dma_k(0);
  if (n > 1) dma_k(1);
  dma_v(0);
  // DMA instructions each wave issues per K (V) stage.
  constexpr int KO = G::KOPS, VO = G::KOPS;
  auto iter_ops = [&](int j) {  // DMA instructions iteration j < n - 1 issues
    if (j == 0) return KO * ((3 < n) + (4 < n)) + VO * (3 < n);
    return KO + VO;
  };

  BfWave<D, NT> w;
  int node[NT], head[NT];
  bool row_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = rb * brows + 32 * (NT * rg + nt) + l32;
    // a row of this block (a padding tile of a 64-row block would be the next block's rows)
    row_ok[nt] = row < a.rows_per_head && (!SPARSE || 32 * (NT * rg + nt) + l32 < block_rows);
    node[nt] = row_ok[nt] ? div_small(row, a.group, a.group_rcp) : 0;
    head[nt] = g * a.group + (row_ok[nt] ? row - node[nt] * a.group : 0);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) w.o[nt][dt] = f32x16{};
    w.m_ref[nt] = kNegInf;
    w.l_run[nt] = 0.f;
    w.alpha[nt] = 1.f;
  }
  w.pend = false;

  // Q, the ancestors and K0 have landed (K1 and V0 may still be on the way):
  // issue K2, V1, V2, then read Q and the ancestor bits, QK(0). Issue order:
  // Q, K0, K1, V0, K2, V1, V2.
  wait_vm_atmost(KO * (n > 1) + VO);
  if (n > 2) dma_k(2);
  if (n > 1) dma_v(1);
  if (n > 2) dma_v(2);
  bf_barrier();
  // The first wave to get here on each SIMD issues its MFMAs before its
  // softmax in every iteration, the second one after (SIMD_ID: HW_ID bits 5:4).
  // (The sparse-block instance runs one real wave per SIMD and has no order
  // to choose.)
  int seen = 0;
  if (!SPARSE && lane == 0) seen = atomicAdd(&s_pair[(__builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11))) & 3], 1);
  // Which of the two takes the MFMA-first order: measured per head dim (the
  // first to arrive for 128, the second for 64; the other way round costs
  // 5% at 70B and 3% on the 64-wide draft shapes).
  const bool mfma_first = (__builtin_amdgcn_readfirstlane(seen) & 1) == (D == 64 ? 1 : 0);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = 32 * (NT * rg + nt) + l32;
    bf_read_k<D>(w.qf[nt], lds0 + (row < 64 ? G::QSTAGE0 : G::QSTAGE1), (row >> 5) & 1, lane);
    // rows past the block's last row (never written out) read node 0's words
    w.anc_at[nt] = lds0 + G::ANC + 8 * (row_ok[nt] ? a.q_first + node[nt] : 0);
  }
  f32x16 sc[NT];
  bf16x8 pp[NT][2];
  bf16x8 vf[2][D / 32];
  if (!idle) {
    bf16x8 kf[D / 16];
    bf_read_k<D>(kf, kslot(0), kh, lane);
    bf_qk<D, NT>(sc, kf, w);
  }
  auto kb_of = [&](int j) { return (t0 + j) * 64 + 32 * kh; };

  // The pipeline, compiled once per order (each copy keeps its own registers).
  auto pipeline = [&](auto order, auto idle_tag, auto free_tag) {
    constexpr bool MF = decltype(order)::value;
    constexpr bool IDLE = decltype(idle_tag)::value;  // loads and barriers only
    constexpr bool FR = decltype(free_tag)::value;    // see bf_iter
    // Iteration 0: softmax(0), QK(1), read V(0); no PV yet. Needs K1 and V0
    // (after V0 come K2, V1, V2).
    wait_vm_atmost(KO * (n > 2) + VO * ((n > 1) + (n > 2)));
    bf_barrier();  // Q has been read by every wave: its staging slots are free
    if (3 < n) dma_k(3);
    if (4 < n) dma_k(4);
    if (3 < n) dma_v(3);
    auto no_dma = [](int) {};
    if constexpr (!IDLE) {
      if (n > 1)
        bf_iter<MF, D, NT, true, false, true, 0, decltype(no_dma)&, FR>(w, sc, pp, vf, kslot(1), vslot(0), kb_of(0), kh, lane, a,
                                                                     no_dma);
      else
        bf_iter<MF, D, NT, false, false, true, 0, decltype(no_dma)&, FR>(w, sc, pp, vf, 0u, vslot(0), kb_of(0), kh, lane, a,
                                                                      no_dma);
    }
    // Steady iteration j: needs K(j+1) and V(j), loads K(j+4) and V(j+3), one
    // DMA instruction after every few MFMAs. Past the split's last stage the
    // loads still run, with an empty range (zeros, no memory traffic), into
    // slots that nothing reads any more (K(j) and V(j-1) are consumed): every
    // steady iteration issues the same instructions, and no branch splits the
    // MFMAs.
    // One buffer range per stream for the whole split, [its first key, the
    // split's end): the stage's offset goes into the per-lane offset, so the
    // range check still zeroes everything past the end, and no descriptor is
    // rebuilt per iteration.
    const int end_keys = min(a.total_keys, t1 * 64);  // loads never reach the next split
    const i32x4 rk = bf_rsrc(kh_ptr + (size_t)t0 * 64 * D, max(end_keys - t0 * 64, 0) * G::ROWB);
    const i32x4 rv = bf_rsrc(vh_ptr + (size_t)t0 * 64 * D, max(end_keys - t0 * 64, 0) * G::ROWB);
    auto steady = [&](int j) {
      const int ko4 = koff + (j + 4) * G::SLOT, vo3 = voff + (j + 3) * G::SLOT;  // G::SLOT: bytes of 64 keys
      const unsigned ks4 = kslot(j + 4);
      const unsigned vs3 = vslot(j + 3);
      auto dma = [&](int i) {
        if (i < G::KOPS) bf_dma16(rk, ks4 + (i * NW + wave) * 1024, ko4, i * NW * 1024);
        else bf_dma16(rv, vs3 + ((i - G::KOPS) * NW + wave) * 1024, vo3, (i - G::KOPS) * NW * 1024);
      };
      if constexpr (IDLE) {
#pragma unroll
        for (int i = 0; i < 2 * G::KOPS; ++i) dma(i);
      } else {
        if constexpr (FR) {
          // A wave alone on its SIMD issues the stage's loads after its
          // iteration (their slots are free all through it): bs = 8 verify
          // 3% faster than with the loads among the MFMAs, which the paired
          // waves of dense blocks keep (70B 2-4% slower the other way).
          bf_iter<MF, D, NT, true, true, true, 0, decltype(no_dma)&, FR>(w, sc, pp, vf, kslot(j + 1), vslot(j),
                                                                        kb_of(j), kh, lane, a, no_dma);
#pragma unroll
          for (int i = 0; i < 2 * G::KOPS; ++i) dma(i);
        } else {
          bf_iter<MF, D, NT, true, true, true, 2 * G::KOPS, decltype(dma)&, FR>(w, sc, pp, vf, kslot(j + 1), vslot(j),
                                                                                kb_of(j), kh, lane, a, dma);
        }
      }
    };
    for (int j = 1; j < n - 1; ++j) {
      // DMA instructions issued after the newest one needed: from j = 3 on,
      // the two previous iterations' (a constant)
      if (j >= 3) {
        static_assert(2 * (KO + VO) <= 15, "vmcnt");
        TA_WAIT_VM(2 * (KO + VO));
      } else {
        wait_vm_atmost(j == 1 ? VO * (n > 2) + iter_ops(0) : (n > 3 ? KO * (n > 4) + VO : 0) + iter_ops(1));
      }
      bf_barrier();
      steady(j);
    }
    // Last iteration (j = n - 1): PV(n-2), softmax(n-1), read V(n-1); no DMA left.
    if (n > 1) {
      TA_WAIT_VM(0);
      bf_barrier();
      if constexpr (!IDLE)
        bf_iter<MF, D, NT, false, true, true, 0, decltype(no_dma)&, FR>(w, sc, pp, vf, 0u, vslot(n - 1), kb_of(n - 1),
                                                                        kh, lane, a, no_dma);
    }
    if constexpr (!IDLE) {
      bf_rescale<D, NT>(w);
      bf_pv<D, NT>(w, vf, pp);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (idle) {
    pipeline(T_{}, T_{}, F_{});
  } else if constexpr (SPARSE) {
    pipeline(T_{}, F_{}, T_{});  // every block sparse: a real wave is alone on its SIMD
  } else {
    if (mfma_first) pipeline(T_{}, F_{}, F_{});
    else pipeline(F_{}, F_{}, F_{});
  }
  __syncthreads();  // every wave is done with the rings: reuse them below

  // Merge the two key halves. The waves of a row group (kh = 0 and 1) each
  // finish half of the head_dim columns: each hands the partner, through
  // LDS in lane order (conflict-free), the other half of its O and its
  // (m, l), then combines and writes out its own half, so all 8 waves share
  // the combine and the stores. Both sides combine in one order, kh = 0's
  // terms first, as one wave combining every column would.
  constexpr int DT = D / 32, HD = DT / 2;  // 32-column blocks of O, half of them per wave
  constexpr int SLOT_F4 = HD * 4 * 64;     // f32x4 of one (tile, key half)'s handed-over columns
  f32x4* xo = reinterpret_cast<f32x4*>(lds);
  float2* xml = reinterpret_cast<float2*>(lds + 8 * SLOT_F4 * 16);
  float l_tot[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) l_tot[nt] = w.l_run[nt] + __shfl_xor(w.l_run[nt], 32);
  auto merge_halves = [&](auto kh_tag) {
    constexpr int KH = decltype(kh_tag)::value;
    constexpr int MINE = KH * HD, THEIRS = (1 - KH) * HD;  // first column block of each half
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int t = NT * rg + nt;
#pragma unroll
      for (int i = 0; i < HD; ++i)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq)
          xo[(t * 2 + KH) * SLOT_F4 + (i * 4 + jq) * 64 + lane] =
              f32x4{w.o[nt][THEIRS + i][4 * jq], w.o[nt][THEIRS + i][4 * jq + 1], w.o[nt][THEIRS + i][4 * jq + 2],
                    w.o[nt][THEIRS + i][4 * jq + 3]};
      if (half == 0) xml[(t * 2 + KH) * 32 + l32] = make_float2(w.m_ref[nt], l_tot[nt]);
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int t = NT * rg + nt;
      const float2 other = xml[(t * 2 + 1 - KH) * 32 + l32];
      const float M = fmaxf(w.m_ref[nt], other.x);
      const float wm = w.m_ref[nt] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(w.m_ref[nt] - M);
      const float wo = other.x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(other.x - M);
      // (weight, values) of key half 0 first
      const float w0 = KH == 0 ? wm : wo, w1 = KH == 0 ? wo : wm;
      w.m_ref[nt] = M;
      l_tot[nt] = KH == 0 ? w0 * l_tot[nt] + w1 * other.y : w0 * other.y + w1 * l_tot[nt];
#pragma unroll
      for (int i = 0; i < HD; ++i)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x4 y = xo[(t * 2 + 1 - KH) * SLOT_F4 + (i * 4 + jq) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float o = w.o[nt][MINE + i][4 * jq + e];
            w.o[nt][MINE + i][4 * jq + e] = KH == 0 ? w0 * o + w1 * y[e] : w0 * y[e] + w1 * o;
          }
        }
    }
    if (a.splits == 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (!row_ok[nt]) continue;
        __bf16* orow = static_cast<__bf16*>(a.out) + ((size_t)node[nt] * a.n_q_heads + head[nt]) * D;
        const float inv = 1.f / l_tot[nt];
#pragma unroll
        for (int i = 0; i < HD; ++i)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const int dt = MINE + i;
            f32x4 x = {w.o[nt][dt][4 * jq], w.o[nt][dt][4 * jq + 1], w.o[nt][dt][4 * jq + 2], w.o[nt][dt][4 * jq + 3]};
            store4<__bf16>(orow + 32 * dt + 8 * jq + 4 * half, x * inv);
          }
      }
    } else {
      // fp32 partials (unnormalised O, reference max, row sum): the merge
      // combines the splits in fp32, so partial outputs of opposite sign
      // cancel without losing digits.
      const PartialSink sink = partial_sink<D>(a, u);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int t = NT * rg + nt;  // 32-row tile of the block
        if (32 * t >= block_rows) continue;  // padding rows: never merged
#pragma unroll
        for (int i = 0; i < HD; ++i)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const int dt = MINE + i;
            put_partial(sink, ((t * DT + dt) * 4 + jq) * 64 + lane,
                        f32x4{w.o[nt][dt][4 * jq], w.o[nt][dt][4 * jq + 1], w.o[nt][dt][4 * jq + 2],
                              w.o[nt][dt][4 * jq + 3]});
          }
        if (KH == 0 && half == 0) put_ml(sink, 32 * t + l32, w.m_ref[nt], l_tot[nt]);
      }
    }
  };
  if (kh == 0) merge_halves(std::integral_constant<int, 0>{});
  else merge_halves(std::integral_constant<int, 1>{});
  if (a.splits == 1) return;
  split_handoff<__bf16, D, kBfThreads<NT>, brows>(a, &s_flags, &s_taken, grp, g, rb, split, tid);
}

}  // namespace

hipError_t launch_tree_attn(const TreeAttnArgs& a, int32_t dtype, int32_t head_dim,
                            hipStream_t stream) {
  const dim3 grid(a.n_units), block(kThreads);
  if (dtype == 1) {
    // 64-row blocks (every head of at most 64 query rows, and the plan's
    // choice where 128-row blocks leave CUs idle): the sparse-block instance
    if (a.block_rows != kBlockRows && a.block_rows != kBlockRows / 2) return hipErrorInvalidValue;
    const bool sparse = a.block_rows == kBlockRows / 2;
    const dim3 bf(kBfThreads<TA_BF16_NT>);
    if (head_dim == 128) {
      if (sparse) hipLaunchKernelGGL((tree_attn_bf16_kernel<128, TA_BF16_NT, true>), grid, bf, 0, stream, a);
      else hipLaunchKernelGGL((tree_attn_bf16_kernel<128, TA_BF16_NT, false>), grid, bf, 0, stream, a);
    } else {
      if (sparse) hipLaunchKernelGGL((tree_attn_bf16_kernel<64, TA_BF16_NT, true>), grid, bf, 0, stream, a);
      else hipLaunchKernelGGL((tree_attn_bf16_kernel<64, TA_BF16_NT, false>), grid, bf, 0, stream, a);
    }
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((tree_attn_kernel<float, 128>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((tree_attn_kernel<float, 64>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ta
