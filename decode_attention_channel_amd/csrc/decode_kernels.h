// Device code of leank_decode_attn: single-token decode attention over the channel-pruned
// cache (LeanK page, section 3.1 item 3 and section 3.2; GQA as in section
// 5.2.3 of the KV-pruning white paper; scale as in FastGen page 5.3).
//
// Work items.  Each (batch row b, KV head h) pair is split into items over
// its full-width rows (K_sl/V_sl, 128 channels) and, for a live head, over
// its middle rows (K_prun with the head's kept channels, V_mid).  One
// 256-thread workgroup runs one item; its 4 wavefronts take the item's row
// tiles round-robin.  All G query heads of the group share every K and V
// load.
//
// Lane layout inside a wavefront (4 rows of 16 lanes):
//   V: lane (r, i) loads 16 bytes (channels 8i..8i+7) of token row 4j + r
//      for V-load j, so a V-load moves 4 whole 256-byte rows.
//   K: a K row of C = 8R channels is loaded by R lanes, 16 bytes each; a
//      K-load moves 64/R rows (1 KB).  Lane (r, i) takes chunk i % R of row
//      4 * (i / R) + r of the load, so the K row that V-load j needs sits in
//      the same 16-lane row r as that V row.
// Scores: bf16 dot2 products of the lane's 8 channels, summed over the R
// lanes of the K row with DPP (quad_perm, half-mirror, mirror), scaled by
// scale*log2(e).  Softmax runs in base 2 with one running max per
// wavefront; the exp2 of each score is computed once in the K layout and
// broadcast to the 16 lanes of its V row with DPP row_newbcast.
//
// Merge.  The 4 rows of a wavefront share the running max, so their sums
// and V accumulators add directly (permlane16/32 swaps).  The 4 wavefronts
// merge through LDS into one (max, sum, acc[G][128]) record per item.  A
// second kernel merges each (b, h) pair's records in item order and writes
// the output, so the result does not depend on scheduling and no workgroup
// waits on another.

// Compile-time tuning knobs (defaults are the measured best on MI355X):
//   LEANK_NT_LOADS         1 = stream K/V with non-temporal loads
//   LEANK_TILE_ROWS_NARROW rows per tile when a K row is <= 32 channels and G <= 4
//   LEANK_TILE_ROWS_WIDE   rows per tile for 64/128-channel K rows and G <= 4

#pragma once

#include <math.h>

#include "common.h"

#ifndef LEANK_NT_LOADS
#define LEANK_NT_LOADS 1
#endif
#ifndef LEANK_TILE_ROWS_NARROW
#define LEANK_TILE_ROWS_NARROW 64
#endif
#ifndef LEANK_TILE_ROWS_WIDE
#define LEANK_TILE_ROWS_WIDE 32
#endif

namespace leank {


constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeHead {
  int64_t k_off;   // elements of K_prun, -1 for a dead head
  int64_t v_off;   // elements of V_mid, -1 for a dead head
  int32_t kept;
  int32_t n_mid;     // middle items of this head per batch row
  int32_t mid_rows;  // rows per middle item
  int32_t base;      // first item of this head within a batch row
};

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_sl;
  const uint16_t* v_sl;
  const uint16_t* k_prun;
  const uint16_t* v_mid;
  const int16_t* kept_idx;
  float* out;
  float* partials;
  int64_t mid_cap;
  int32_t n_kv;
  int32_t n_q;
  int32_t slots;
  int32_t t_sl;
  int32_t t_mid;
  int32_t n_sl_items;
  int32_t sl_rows;
  int32_t items_per_b;
  int32_t partial_stride;
  int32_t combine_slices;  // channel slices per (pair, query head) in the combine
  float qk_scale;  // softmax scale * log2(e)
  DecodeHead heads[LEANK_MAX_KV_HEADS];
};

// The running max only moves when a tile's max exceeds it by more than this
// (base-2 units), so weights stay <= 2^kRescaleSlack and most tiles skip
// the rescale; the softmax is unchanged because the reference cancels.
constexpr float kRescaleSlack = 8.0f;

template <int G>
struct Running {
  float m[G];       // reference max (base-2 units), uniform over the wavefront
  float l[G];       // sum of exp2 weights of this lane's K rows (K layout)
  float acc[G][8];  // weighted V for this lane's 8 channels (V layout)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x + x of the row at lane distance 16 / 32, as a VALU swap (no LDS).
__device__ __forceinline__ float add_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of streamed cache data (read once per call).
__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
#if LEANK_NT_LOADS
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#else
  const u32x4_t t = *reinterpret_cast<const u32x4_t*>(p);
#endif
  return make_uint4(t[0], t[1], t[2], t[3]);
}

template <int G, int R>
struct TileShape {
  static constexpr int kRowsPerKLoad = 64 / R;
  static constexpr int kWant =
      G > 4 ? (R == 16 ? 16 : 32) : (R >= 8 ? LEANK_TILE_ROWS_WIDE : LEANK_TILE_ROWS_NARROW);
  static constexpr int kRows = kWant > kRowsPerKLoad ? kWant : kRowsPerKLoad;
  static constexpr int kVLoads = kRows / 4;
  static constexpr int kKLoads = kRows / kRowsPerKLoad;
  static constexpr int kRowsPerGroup = 16 / R;  // K rows per 16-lane row per K-load
};

// One tile of kRows rows starting at row t0 of the stream (rows >= nvalid
// are outside the item when kTail).  kb/vb point at row 0 of the K and V
// streams; kstride is the K row length in elements (= 8R unless kGeneric,
// where R = 16 and only lanes with k_active hold K data).
template <int G, int R, bool kTail, bool kGeneric>
__device__ __forceinline__ void attend_tile(const uint16_t* __restrict__ kb,
                                            const uint16_t* __restrict__ vb, int kstride, int t0,
                                            int nvalid, bool k_active, const uint32_t (&qw)[G][4],
                                            float qk_scale, Running<G>& st) {
  using S = TileShape<G, R>;
  const int lane = threadIdx.x & 63;
  const int row16 = lane >> 4;
  const int i = lane & 15;
  const int grp = i / R;
  const int chunk = i % R;

  const uint16_t* kt = kb + static_cast<int64_t>(t0) * kstride;
  const uint16_t* vt = vb + static_cast<int64_t>(t0) * LEANK_HEAD_DIM;
  uint4 kv[S::kKLoads];
  uint4 vv[S::kVLoads];
  static_for<S::kKLoads>([&](auto KK) {
    constexpr int kk = decltype(KK)::value;
    const int row = kk * S::kRowsPerKLoad + 4 * grp + row16;
    const bool ok = (!kTail || row < nvalid) && (!kGeneric || k_active);
    kv[kk] = ok ? load_stream16(kt + row * kstride + chunk * 8) : make_uint4(0u, 0u, 0u, 0u);
  });
  static_for<S::kVLoads>([&](auto JJ) {
    constexpr int jj = decltype(JJ)::value;
    const int row = 4 * jj + row16;
    const bool ok = !kTail || row < nvalid;
    vv[jj] = ok ? load_stream16(vt + row * LEANK_HEAD_DIM + i * 8) : make_uint4(0u, 0u, 0u, 0u);
  });

  // scores (base-2 logits) of the K rows this lane's group holds
  float s[S::kKLoads][G];
  static_for<S::kKLoads>([&](auto KK) {
    constexpr int kk = decltype(KK)::value;
    const int row = kk * S::kRowsPerKLoad + 4 * grp + row16;
    static_for<G>([&](auto GG) {
      constexpr int g = decltype(GG)::value;
      float a = dot2_bf16(qw[g][0], kv[kk].x, 0.0f);
      a = dot2_bf16(qw[g][1], kv[kk].y, a);
      a = dot2_bf16(qw[g][2], kv[kk].z, a);
      a = dot2_bf16(qw[g][3], kv[kk].w, a);
      if constexpr (R >= 2) a += dpp_f32<kDppQuadXor1>(a);
      if constexpr (R >= 4) a += dpp_f32<kDppQuadXor2>(a);
      if constexpr (R >= 8) a += dpp_f32<kDppHalfMirror>(a);
      if constexpr (R >= 16) a += dpp_f32<kDppRowMirror>(a);
      a *= qk_scale;
      if (kTail && row >= nvalid) a = -INFINITY;
      s[kk][g] = a;
    });
  });

  // running max over the wavefront, lazy rescale, exp2 in the K layout
  static_for<G>([&](auto GG) {
    constexpr int g = decltype(GG)::value;
    float mx = s[0][g];
    static_for<S::kKLoads>([&](auto KK) {
      constexpr int kk = decltype(KK)::value;
      if constexpr (kk > 0) mx = fmaxf(mx, s[kk][g]);
    });
    if constexpr (R < 2) mx = fmaxf(mx, dpp_f32<kDppQuadXor1>(mx));
    if constexpr (R < 4) mx = fmaxf(mx, dpp_f32<kDppQuadXor2>(mx));
    if constexpr (R < 8) mx = fmaxf(mx, dpp_f32<kDppHalfMirror>(mx));
    if constexpr (R < 16) mx = fmaxf(mx, dpp_f32<kDppRowMirror>(mx));
    mx = max_xor32(max_xor16(mx));
    mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));
    if (mx > st.m[g] + kRescaleSlack) {  // uniform over the wavefront
      const float corr = st.m[g] == -INFINITY ? 0.0f : fast_exp2(st.m[g] - mx);
      st.m[g] = mx;
      st.l[g] *= corr;
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] *= corr;
    }
    const float m_use = st.m[g] == -INFINITY ? 0.0f : st.m[g];
    static_for<S::kKLoads>([&](auto KK) {
      constexpr int kk = decltype(KK)::value;
      s[kk][g] = fast_exp2(s[kk][g] - m_use);
      st.l[g] += s[kk][g];
    });
  });

  // weighted V: V-load jj holds row 4jj + row16, whose weight sits in K-load
  // jj / kRowsPerGroup, lane group jj % kRowsPerGroup of the same 16-lane row
  static_for<S::kVLoads>([&](auto JJ) {
    constexpr int jj = decltype(JJ)::value;
    constexpr int kk = jj / S::kRowsPerGroup;
    constexpr int src_lane = R * (jj % S::kRowsPerGroup);
    float v[8];
    v[0] = bf16_lo(vv[jj].x);
    v[1] = bf16_hi(vv[jj].x);
    v[2] = bf16_lo(vv[jj].y);
    v[3] = bf16_hi(vv[jj].y);
    v[4] = bf16_lo(vv[jj].z);
    v[5] = bf16_hi(vv[jj].z);
    v[6] = bf16_lo(vv[jj].w);
    v[7] = bf16_hi(vv[jj].w);
    static_for<G>([&](auto GG) {
      constexpr int g = decltype(GG)::value;
      float p;
      if constexpr (S::kRowsPerGroup == 1) {
        p = s[kk][g];
      } else {
        p = dpp_f32<kDppRowNewBcast + src_lane>(s[kk][g]);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] = fmaf(p, v[c], st.acc[g][c]);
    });
  });
}

template <int G, int R, bool kGeneric>
__device__ __forceinline__ void attend_range(const uint16_t* kb, const uint16_t* vb, int kstride,
                                             int r0, int r1, bool k_active,
                                             const uint32_t (&qw)[G][4], float qk_scale,
                                             Running<G>& st) {
  constexpr int kRows = TileShape<G, R>::kRows;
  const int wave = threadIdx.x >> 6;
  for (int t0 = r0 + wave * kRows; t0 < r1; t0 += kWaves * kRows) {
    const int nvalid = r1 - t0;
    if (nvalid >= kRows) {
      attend_tile<G, R, false, kGeneric>(kb, vb, kstride, t0, kRows, k_active, qw, qk_scale, st);
    } else {
      attend_tile<G, R, true, kGeneric>(kb, vb, kstride, t0, nvalid, k_active, qw, qk_scale, st);
    }
  }
  // each lane group of R lanes summed the weights of its own K rows: add the
  // groups of the 16-lane row so that l covers the row's V rows like acc
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (R < 2) st.l[g] += dpp_f32<kDppQuadXor1>(st.l[g]);
    if constexpr (R < 4) st.l[g] += dpp_f32<kDppQuadXor2>(st.l[g]);
    if constexpr (R < 8) st.l[g] += dpp_f32<kDppHalfMirror>(st.l[g]);
    if constexpr (R < 16) st.l[g] += dpp_f32<kDppRowMirror>(st.l[g]);
  }
}

// q channels of the lane's K chunk for the G query heads, packed bf16 pairs.
template <int G>
__device__ __forceinline__ void load_q_dense(const uint16_t* qh, int chunk, uint32_t (&qw)[G][4]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 w = *reinterpret_cast<const uint4*>(qh + g * LEANK_HEAD_DIM + chunk * 8);
    qw[g][0] = w.x;
    qw[g][1] = w.y;
    qw[g][2] = w.z;
    qw[g][3] = w.w;
  }
}

template <int G>
__device__ __forceinline__ void load_q_gather(const uint16_t* qh, const int16_t* idx, int chunk,
                                              bool active, uint32_t (&qw)[G][4]) {
  int ch[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) ch[k] = active ? (idx[chunk * 8 + k] & (LEANK_HEAD_DIM - 1)) : 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = active ? qh[g * LEANK_HEAD_DIM + ch[2 * k]] : 0u;
      const uint32_t hi = active ? qh[g * LEANK_HEAD_DIM + ch[2 * k + 1]] : 0u;
      qw[g][k] = lo | (hi << 16);
    }
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeParams p) {
  __shared__ float s_acc[kWaves][G][LEANK_HEAD_DIM];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];

  const int item = blockIdx.x;
  const int b = item / p.items_per_b;
  const int r = item - b * p.items_per_b;
  int h = 0;
  while (h + 1 < p.n_kv && r >= p.heads[h + 1].base) ++h;
  const DecodeHead hd = p.heads[h];
  const int local = r - hd.base;
  const bool middle = local >= p.n_sl_items;

  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const uint16_t* qh = p.q + (static_cast<int64_t>(b) * p.n_q + h * G) * LEANK_HEAD_DIM;

  Running<G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.acc[g][c] = 0.0f;
  }
  uint32_t qw[G][4];

  if (!middle) {
    const int r0 = local * p.sl_rows;
    const int r1 = min(p.t_sl, r0 + p.sl_rows);
    const int64_t pair = static_cast<int64_t>(b) * p.n_kv + h;
    const uint16_t* kb = p.k_sl + pair * p.slots * LEANK_HEAD_DIM;
    const uint16_t* vb = p.v_sl + pair * p.slots * LEANK_HEAD_DIM;
    load_q_dense<G>(qh, i, qw);
    attend_range<G, 16, false>(kb, vb, LEANK_HEAD_DIM, r0, r1, true, qw, p.qk_scale, st);
  } else {
    const int chunk_id = local - p.n_sl_items;
    const int r0 = chunk_id * hd.mid_rows;
    const int r1 = min(p.t_mid, r0 + hd.mid_rows);
    const int kept = hd.kept;
    const int64_t brow = static_cast<int64_t>(b) * p.mid_cap;
    const uint16_t* kb = p.k_prun + hd.k_off + brow * kept;
    const uint16_t* vb = p.v_mid + hd.v_off + brow * LEANK_HEAD_DIM;
    const int16_t* idx = p.kept_idx + h * LEANK_HEAD_DIM;
    switch (kept) {
      case 8:
        load_q_gather<G>(qh, idx, i % 1, true, qw);
        attend_range<G, 1, false>(kb, vb, 8, r0, r1, true, qw, p.qk_scale, st);
        break;
      case 16:
        load_q_gather<G>(qh, idx, i % 2, true, qw);
        attend_range<G, 2, false>(kb, vb, 16, r0, r1, true, qw, p.qk_scale, st);
        break;
      case 32:
        load_q_gather<G>(qh, idx, i % 4, true, qw);
        attend_range<G, 4, false>(kb, vb, 32, r0, r1, true, qw, p.qk_scale, st);
        break;
      case 64:
        load_q_gather<G>(qh, idx, i % 8, true, qw);
        attend_range<G, 8, false>(kb, vb, 64, r0, r1, true, qw, p.qk_scale, st);
        break;
      case 128:
        load_q_gather<G>(qh, idx, i, true, qw);
        attend_range<G, 16, false>(kb, vb, 128, r0, r1, true, qw, p.qk_scale, st);
        break;
      default: {
        const bool active = i < kept / 8;
        load_q_gather<G>(qh, idx, i, active, qw);
        attend_range<G, 16, true>(kb, vb, kept, r0, r1, active, qw, p.qk_scale, st);
        break;
      }
    }
  }

  // the 4 rows of the wavefront share st.m: add their sums and accumulators
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.l[g] = add_xor32(add_xor16(st.l[g]));
#pragma unroll
    for (int c = 0; c < 8; ++c) st.acc[g][c] = add_xor32(add_xor16(st.acc[g][c]));
  }
  const int wave = threadIdx.x >> 6;
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s_acc[wave][g][lane * 8 + c] = st.acc[g][c];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_m[wave][g] = st.m[g];
      s_l[wave][g] = st.l[g];
    }
  }
  __syncthreads();

  // one record per item: (acc[G][128], m[G], l[G]) merged over the wavefronts
  float* rec = p.partials + static_cast<int64_t>(item) * p.partial_stride;
  for (int t = threadIdx.x; t < G * LEANK_HEAD_DIM; t += kThreads) {
    const int g = t / LEANK_HEAD_DIM;
    const int ch = t - g * LEANK_HEAD_DIM;
    float m = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_m[w][g]);
    const float m_use = m == -INFINITY ? 0.0f : m;
    float a = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][g] - m_use);
      a = fmaf(s_acc[w][g][ch], f, a);
      l = fmaf(s_l[w][g], f, l);
    }
    rec[t] = a;
    if (ch == 0) {
      rec[G * LEANK_HEAD_DIM + g] = m;
      rec[G * LEANK_HEAD_DIM + G + g] = l;
    }
  }
}

// Merges the records of one (batch row, KV head) pair for one query head g
// of its group -- or, when the pair has many items, for one of `slices`
// channel slices of that head -- and writes the output.  Threads form
// item groups x float4 channel quads; item group j takes items j, j+groups,
// ...; the groups are summed in a fixed order, so the result does not
// depend on timing.  Grid: pairs x G x slices.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(const DecodeParams p) {
  __shared__ float s_max[kThreads];
  __shared__ float4 s_acc[kThreads];
  __shared__ float s_sum[kThreads];
  const int slices = p.combine_slices;
  const int quads = LEANK_HEAD_DIM / 4 / slices;  // float4 quads per workgroup
  const int groups = kThreads / quads;
  int64_t rest = blockIdx.x;
  const int slice = static_cast<int>(rest % slices);
  rest /= slices;
  const int g = static_cast<int>(rest % G);
  const int64_t pair = rest / G;
  const int b = static_cast<int>(pair / p.n_kv);
  const int h = static_cast<int>(pair - static_cast<int64_t>(b) * p.n_kv);
  const DecodeHead hd = p.heads[h];
  const int n_items = p.n_sl_items + hd.n_mid;
  const int64_t stride = p.partial_stride;
  const float* first = p.partials + (static_cast<int64_t>(b) * p.items_per_b + hd.base) * stride;
  const int m_off = G * LEANK_HEAD_DIM + g;
  const int l_off = G * LEANK_HEAD_DIM + G + g;
  const int t = threadIdx.x;

  float m = -INFINITY;
  for (int n = t; n < n_items; n += kThreads) m = fmaxf(m, first[n * stride + m_off]);
  s_max[t] = m;
  __syncthreads();
  for (int half = kThreads / 2; half > 0; half /= 2) {
    if (t < half) s_max[t] = fmaxf(s_max[t], s_max[t + half]);
    __syncthreads();
  }
  const float m_all = s_max[0];
  const float m_use = m_all == -INFINITY ? 0.0f : m_all;

  const int grp = t / quads;
  const int quad = t - grp * quads;
  const int ch = g * LEANK_HEAD_DIM + (slice * quads + quad) * 4;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float l = 0.0f;
  int n = grp;
  for (; n + 3 * groups < n_items; n += 4 * groups) {
    float f[4], lw[4];
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* rn = first + (n + u * groups) * stride;
      f[u] = rn[m_off];
      lw[u] = rn[l_off];
      v[u] = *reinterpret_cast<const float4*>(rn + ch);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = fast_exp2(f[u] - m_use);
      a.x = fmaf(v[u].x, w, a.x);
      a.y = fmaf(v[u].y, w, a.y);
      a.z = fmaf(v[u].z, w, a.z);
      a.w = fmaf(v[u].w, w, a.w);
      l = fmaf(lw[u], w, l);
    }
  }
  for (; n < n_items; n += groups) {
    const float* rn = first + n * stride;
    const float w = fast_exp2(rn[m_off] - m_use);
    const float4 v = *reinterpret_cast<const float4*>(rn + ch);
    a.x = fmaf(v.x, w, a.x);
    a.y = fmaf(v.y, w, a.y);
    a.z = fmaf(v.z, w, a.z);
    a.w = fmaf(v.w, w, a.w);
    l = fmaf(rn[l_off], w, l);
  }
  s_acc[t] = a;
  s_sum[t] = l;
  __syncthreads();
  if (t < quads) {
    float4 o = s_acc[t];
    float total = s_sum[t];
    for (int j = 1; j < groups; ++j) {
      const float4 x = s_acc[j * quads + t];
      o.x += x.x;
      o.y += x.y;
      o.z += x.z;
      o.w += x.w;
      total += s_sum[j * quads + t];
    }
    const float inv = 1.0f / total;
    float* out = p.out + (static_cast<int64_t>(b) * p.n_q + h * G) * LEANK_HEAD_DIM + ch;
    *reinterpret_cast<float4*>(out) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

// Launches the split and combine kernels for G query heads per KV head.
template <int G>
int launch_decode(const DecodeParams& p, int64_t n_items, int64_t n_pairs, hipStream_t s) {
  hipLaunchKernelGGL(decode_split_kernel<G>, dim3(static_cast<unsigned>(n_items)), dim3(kThreads),
                     0, s, p);
  LEANK_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(decode_combine_kernel<G>,
                     dim3(static_cast<unsigned>(n_pairs * G * p.combine_slices)), dim3(kThreads),
                     0, s, p);
  LEANK_HIP_TRY(hipGetLastError());
  return LEANK_OK;
}

}  // namespace leank
