// Tree-masked attention for gfx950 (CDNA4).
//
// What is computed (SwiftSpec, arXiv 2506.11309, Pith review page, "What
// carries the argument" and the referee summary): each tree token attends to
// the verified prefix, to its ancestors in the tree and to itself; the cache
// holds the prefix contiguously with the tree tokens right after it. The
// pages' kernel targets Hopper and hands partial results between thread
// blocks without explicit barriers; here the same idea is a per-row-block
// arrival counter (release/acquire at agent scope) and the last workgroup to
// arrive merges the split results, so the whole call is one launch with no
// grid barrier.
//
// Work decomposition. One workgroup = 4 waves = 128 query rows of one KV head
// (row r of a head is tree node r / G, query head g*G + r % G, so a GQA
// group's rows share every K/V tile) times one contiguous range of 32-key
// tiles (a "split" of [0, prefix_len + n_tree)). Splits exist to spread a few
// KV heads over 256 CUs; their partial (max, sum, unnormalised output) rows go
// to the workspace and are merged in split order, so results are
// deterministic for a given shape.
//
// Per tile: K (32 x D, row-major) and V (transposed to D x 32, keys permuted to
// match the MFMA operand layout) are staged in LDS by all 256 threads; the
// next tile's global loads are in flight while the current one is consumed.
// Each wave computes S^T = K Q^T with MFMA (keys = M, its 32 rows = N,
// head_dim = K), so after the product every lane holds 16 scores of ONE row:
// the online softmax needs only a single cross-lane exchange (lane ^ 32) per
// tile. Then O^T += V^T P^T with MFMA, whose accumulator again holds one row
// per lane, so the running-max rescale is a per-lane scalar.
//
// Ancestor mask: one 64-bit word per row (bit j = tree node j visible), held
// in a register; only tiles that reach past the prefix test it.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "launch.h"

namespace ta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 32;
constexpr int kBlockRows = 128;
constexpr float kNegInf = -__builtin_huge_valf();

// Position of key `k` (0..31) inside a transposed V row in LDS. The PV MFMA
// reads, per lane half and k-slot, the keys that the S^T accumulator gave that
// lane; this permutation makes those keys contiguous so one wide LDS read
// fetches a whole operand.
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

template <typename T, int D>
struct Layout {
  static constexpr int ES = sizeof(T);
  static constexpr int KSTR = D * ES + 16;        // K row stride in LDS (bytes)
  static constexpr int VSTR = kTile * ES + 16;    // transposed V row stride
  static constexpr int KBYTES = kTile * KSTR;
  static constexpr int BUF = KBYTES + D * VSTR;   // one stage
  static constexpr int KCHUNKS = kTile * D * ES / 16;       // 16-B chunks per K tile
  static constexpr int KREP = (KCHUNKS + kThreads - 1) / kThreads;
  static constexpr int VE = 8 / ES;                         // d values per 8-B V read
  static constexpr int VBLOCKS = (kTile / 4) * (D / VE);    // 4 keys x VE d blocks
  static constexpr int VREP = (VBLOCKS + kThreads - 1) / kThreads;
};

template <typename T, int D>
struct Stage {
  uint4 kreg[Layout<T, D>::KREP];
  uint2 vreg[Layout<T, D>::VREP][4];
};

// Global -> registers for tile `tile`. Keys at or beyond total_keys load as 0
// and are never read from memory.
template <typename T, int D>
__device__ __forceinline__ void load_tile(Stage<T, D>& st, const T* kh, const T* vh, int tile,
                                          int total_keys, int tid) {
  using L = Layout<T, D>;
  constexpr int CPR = D * L::ES / 16;  // 16-B chunks per K row
#pragma unroll
  for (int r = 0; r < L::KREP; ++r) {
    const int ci = tid + r * kThreads;
    const int key = ci / CPR, col = ci % CPR;
    const int gk = tile * kTile + key;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (ci < L::KCHUNKS && gk < total_keys)
      x = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(kh + (size_t)gk * D) + col * 16);
    st.kreg[r] = x;
  }
  constexpr int DG = D / L::VE;  // d groups per key row
#pragma unroll
  for (int r = 0; r < L::VREP; ++r) {
    const int bi = tid + r * kThreads;
    const int dg = bi % DG, kg = bi / DG;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int gk = tile * kTile + kg * 4 + b;
      uint2 x = make_uint2(0, 0);
      if (bi < L::VBLOCKS && gk < total_keys)
        x = *reinterpret_cast<const uint2*>(vh + (size_t)gk * D + dg * L::VE);
      st.vreg[r][b] = x;
    }
  }
}

// Registers -> LDS stage: K row-major, V transposed with keys permuted.
template <typename T, int D>
__device__ __forceinline__ void store_tile(const Stage<T, D>& st, char* buf, int tid) {
  using L = Layout<T, D>;
  constexpr int CPR = D * L::ES / 16;
#pragma unroll
  for (int r = 0; r < L::KREP; ++r) {
    const int ci = tid + r * kThreads;
    if (ci < L::KCHUNKS)
      *reinterpret_cast<uint4*>(buf + (ci / CPR) * L::KSTR + (ci % CPR) * 16) = st.kreg[r];
  }
  char* vt = buf + L::KBYTES;
  constexpr int DG = D / L::VE;
#pragma unroll
  for (int r = 0; r < L::VREP; ++r) {
    const int bi = tid + r * kThreads;
    if (bi >= L::VBLOCKS) continue;
    const int dg = bi % DG, kg = bi / DG;
    const int col = vpos<T>(kg * 4) * L::ES;  // 4 consecutive keys stay contiguous
    if constexpr (std::is_same_v<T, float>) {
      // 2 d values per key row; write 4 keys (16 B) per d.
      const uint2* x = st.vreg[r];
      *reinterpret_cast<uint4*>(vt + (dg * 2 + 0) * L::VSTR + col) = make_uint4(x[0].x, x[1].x, x[2].x, x[3].x);
      *reinterpret_cast<uint4*>(vt + (dg * 2 + 1) * L::VSTR + col) = make_uint4(x[0].y, x[1].y, x[2].y, x[3].y);
    } else {
      // 4 d values per key row; write 4 keys (8 B) per d (a 4x4 16-bit transpose).
      const uint2* x = st.vreg[r];
      const uint32_t lo01 = (x[0].x & 0xFFFFu) | (x[1].x << 16);
      const uint32_t lo23 = (x[2].x & 0xFFFFu) | (x[3].x << 16);
      const uint32_t hi01 = (x[0].x >> 16) | (x[1].x & 0xFFFF0000u);
      const uint32_t hi23 = (x[2].x >> 16) | (x[3].x & 0xFFFF0000u);
      const uint32_t lo01y = (x[0].y & 0xFFFFu) | (x[1].y << 16);
      const uint32_t lo23y = (x[2].y & 0xFFFFu) | (x[3].y << 16);
      const uint32_t hi01y = (x[0].y >> 16) | (x[1].y & 0xFFFF0000u);
      const uint32_t hi23y = (x[2].y >> 16) | (x[3].y & 0xFFFF0000u);
      *reinterpret_cast<uint2*>(vt + (dg * 4 + 0) * L::VSTR + col) = make_uint2(lo01, lo23);
      *reinterpret_cast<uint2*>(vt + (dg * 4 + 1) * L::VSTR + col) = make_uint2(hi01, hi23);
      *reinterpret_cast<uint2*>(vt + (dg * 4 + 2) * L::VSTR + col) = make_uint2(lo01y, lo23y);
      *reinterpret_cast<uint2*>(vt + (dg * 4 + 3) * L::VSTR + col) = make_uint2(hi01y, hi23y);
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
  const char* krow = kbuf + l32 * L::KSTR;
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

// O^T (D x 32 rows) += V^T P^T for one tile; p[j] pairs with the key layout of qk_tile.
template <typename T, int D>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[D / 32], const float (&p)[16], const char* vbuf,
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

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void tree_attn_kernel(const TreeAttnArgs a) {
  using L = Layout<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::BUF];
  __shared__ int s_last;

  // Work unit. Consecutive workgroup ids go round-robin over the 8 XCDs, so
  // give each XCD a contiguous run of units: the row blocks and splits of one
  // KV head then share that XCD's L2.
  const int b = blockIdx.x;
  const int u = (a.n_units % 8 == 0) ? (b % 8) * (a.n_units / 8) + b / 8 : b;
  const int split = u % a.splits;
  const int grp = u / a.splits;  // (KV head, row block)
  const int rb = grp % a.row_blocks;
  const int g = grp / a.row_blocks;
  const int t0 = (int)((long long)split * a.n_tiles / a.splits);
  const int t1 = (int)((long long)(split + 1) * a.n_tiles / a.splits);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int rloc = wave * 32 + l32;          // row within the block
  const int row = rb * kBlockRows + rloc;    // row within the KV head
  const bool row_ok = row < a.rows_per_head;
  const int node = row_ok ? row / a.group : 0;
  const int head = g * a.group + (row_ok ? row % a.group : 0);
  const uint64_t anc = row_ok ? a.anc[node] : 0;

  const T* kh = static_cast<const T*>(a.k) + (size_t)g * a.kv_head_stride;
  const T* vh = static_cast<const T*>(a.v) + (size_t)g * a.kv_head_stride;

  QFrag<T, D> qf;
  load_q<T, D>(qf, static_cast<const T*>(a.q) + ((size_t)node * a.n_q_heads + head) * D, row_ok, half);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  Stage<T, D> st;
  load_tile<T, D>(st, kh, vh, t0, a.total_keys, tid);
  store_tile<T, D>(st, smem, tid);
  __syncthreads();

  for (int tile = t0; tile < t1; ++tile) {
    char* cur = smem + ((tile - t0) & 1) * L::BUF;
    const bool more = tile + 1 < t1;
    if (more) load_tile<T, D>(st, kh, vh, tile + 1, a.total_keys, tid);

    const f32x16 s = qk_tile<T, D>(qf, cur, l32, half);
    const int kb = tile * kTile;
    float p[16];
    float mx = kNegInf;
    if (kb + kTile > a.prefix_len) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kb + 8 * (j >> 2) + 4 * half + (j & 3);
        bool vis = key < a.prefix_len;
        if (!vis && key < a.total_keys) vis = (anc >> (key - a.prefix_len)) & 1;
        p[j] = vis ? s[j] * a.scale_log2 : kNegInf;
        mx = fmaxf(mx, p[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        p[j] = s[j] * a.scale_log2;
        mx = fmaxf(mx, p[j]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;  // fully masked so far
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[j] = __builtin_amdgcn_exp2f(p[j] - m_use);
      psum += p[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    }
    pv_tile<T, D>(o, p, cur + L::KBYTES, l32, half);

    if (more) store_tile<T, D>(st, smem + ((tile + 1 - t0) & 1) * L::BUF, tid);
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

  // Split: publish this split's partial rows, then take a ticket.
  {
    float* po = a.ws_o + ((size_t)u * kBlockRows + rloc) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        f32x4 x = {o[dt][4 * jq], o[dt][4 * jq + 1], o[dt][4 * jq + 2], o[dt][4 * jq + 3]};
        *reinterpret_cast<f32x4*>(po + 32 * dt + 8 * jq + 4 * half) = x;
      }
    if (half == 0) a.ws_ml[(size_t)u * kBlockRows + rloc] = make_float2(m_run, l_tot);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(a.ws_cnt + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == a.splits - 1;
    if (last) __hip_atomic_store(a.ws_cnt + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // Last arrival: merge the splits of this row block, in split order.
  const size_t u0 = (size_t)grp * a.splits;
  constexpr int C4 = D / 4;  // float4 chunks per row
  for (int item = tid; item < kBlockRows * C4; item += kThreads) {
    const int r = item / C4, c = item % C4;
    const int hrow = rb * kBlockRows + r;
    if (hrow >= a.rows_per_head) continue;
    float M = kNegInf;
    for (int s2 = 0; s2 < a.splits; ++s2) M = fmaxf(M, a.ws_ml[(u0 + s2) * kBlockRows + r].x);
    float Lsum = 0.f;
    f32x4 acc = {0, 0, 0, 0};
    for (int s2 = 0; s2 < a.splits; ++s2) {
      const float2 ml = a.ws_ml[(u0 + s2) * kBlockRows + r];
      const float w = ml.x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
      Lsum += w * ml.y;
      acc += w * *reinterpret_cast<const f32x4*>(a.ws_o + ((u0 + s2) * kBlockRows + r) * D + 4 * c);
    }
    const int nd = hrow / a.group;
    const int hd = g * a.group + hrow % a.group;
    store4<T>(static_cast<T*>(a.out) + ((size_t)nd * a.n_q_heads + hd) * D + 4 * c, acc * (1.f / Lsum));
  }
}

}  // namespace

hipError_t launch_tree_attn(const TreeAttnArgs& a, int32_t dtype, int32_t head_dim,
                            hipStream_t stream) {
  const dim3 grid(a.n_units), block(kThreads);
  if (dtype == 1) {
    if (head_dim == 128)
      hipLaunchKernelGGL((tree_attn_kernel<__bf16, 128>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((tree_attn_kernel<__bf16, 64>), grid, block, 0, stream, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((tree_attn_kernel<float, 128>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((tree_attn_kernel<float, 64>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ta
