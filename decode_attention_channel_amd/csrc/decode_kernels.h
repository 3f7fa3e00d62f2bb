// Device code of leank_decode_attn: single-token decode attention over the
// channel-pruned cache (LeanK page, section 3.1 item 3 and section 3.2; GQA
// as in section 5.2.3 of the KV-pruning white paper; scale as in FastGen
// page 5.3).
//
// Work items.  Each (batch row b, KV head h) pair is split into items over
// its full-width rows (K_sl/V_sl, 128 channels) and, for a live head, over
// its middle rows (K_prun with the head's kept channels c, V_mid).  One
// 256-thread workgroup runs one item; its 4 wavefronts take 32-row tiles
// round-robin.  All G query heads of the group share every K and V load.
//
// Matrix instructions (v_mfma_f32_16x16x32_bf16; lane l, col = l % 16,
// grp = l / 16):
//   scores  S[head][row] = Q[head][ch] K[row][ch]^T: the A operand is the
//           group's q (head = col, 8 channels per lane, gathered through
//           kept_idx), the B operand is K as stored (row = col, the same 8
//           channels: one 16-byte load of a K row), one instruction per 16
//           rows and 32 channels;
//   output  O[head][ch] += P[head][row] V[row][ch]: the A operand is P
//           (head = col, rows 8 grp .. 8 grp + 7), the B operand is V as
//           stored in 8-row blocks (channel = col, one 16-byte load = the
//           8 rows), one instruction per 32 rows and 16 channels.  P goes
//           in as two bf16 parts (hi + lo), which keeps about 16 bits of
//           each weight.
// Results of both land with head 4 grp + i in register i, so the softmax of
// a head runs inside one 16-lane row: DPP reductions only, base-2 exp of
// scores pre-scaled by scale * log2(e), and a reference max that moves only
// when a tile's max exceeds it by more than 2^8.  P reaches the A-operand
// layout through a 2 KiB per-wavefront LDS transpose.
//
// Merge.  The 4 wavefronts merge through LDS into one (max, sum,
// acc[G][128]) record per item.  A second kernel merges each (b, h) pair's
// records in item order and writes the output, so the result does not
// depend on scheduling and no workgroup waits on another.
//
// Compile-time tuning knobs (defaults are the measured best on MI355X):
//   LEANK_NT_LOADS      1 = stream K/V with non-temporal loads
//   LEANK_PREFETCH      1 = load the next tile while the current one computes
//   LEANK_WAVES_PER_EU  register budget hint for the split kernel (0 = none)

#pragma once

#include <math.h>

#include "common.h"
#include "quant.h"

#ifndef LEANK_NT_LOADS
#define LEANK_NT_LOADS 1
#endif
#ifndef LEANK_PREFETCH
#define LEANK_PREFETCH 0
#endif
#ifndef LEANK_WAVES_PER_EU
#define LEANK_WAVES_PER_EU 3
#endif
#ifndef LEANK_Q_WAVES_PER_EU
#define LEANK_Q_WAVES_PER_EU 2
#endif
// register budget: LEANK_WAVES_PER_EU for bf16 caches and for low-bit
// middle streams whose live heads keep at most 32 channels;
// LEANK_Q_WAVES_PER_EU for wider low-bit heads (dequantizing more channel
// blocks keeps more registers live)
#if LEANK_WAVES_PER_EU
#define LEANK_SPLIT_ATTRS                  \
  __launch_bounds__(kThreads) __attribute__( \
      (amdgpu_waves_per_eu(QB && KBMAX > 1 ? LEANK_Q_WAVES_PER_EU : LEANK_WAVES_PER_EU)))
#else
#define LEANK_SPLIT_ATTRS __launch_bounds__(kThreads)
#endif

namespace leank {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileRows = 32;
constexpr float kLog2e = 1.4426950408889634f;

// The reference max only moves when a tile's max exceeds it by more than
// this (base-2 units), so weights stay <= 2^kRescaleSlack and most tiles
// skip the rescale; the softmax is unchanged because the reference cancels.
constexpr float kRescaleSlack = 8.0f;

struct DecodeHead {
  int64_t k_off;   // elements of K_prun, -1 for a dead head (low-bit: kept channels of the live heads before it)
  int64_t v_off;   // elements of V_mid, -1 for a dead head (low-bit: its rank among the live heads)
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
  const int32_t* ctx_lens;  // per-row context lengths (ragged batches), or null
  // fused decode step: the appended token's K and V [B][H_kv][128], and its
  // position per row (row_pos, ragged) or for every row (step_pos)
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int64_t* row_pos;
  int64_t step_pos;
  int64_t mid_cap;
  int64_t v_mid_rows;  // stored V rows per batch row of a middle segment
  int64_t v_sl_rows;   // stored V rows per (batch row, head) of the ring
  int32_t n_kv;
  int32_t n_q;
  int32_t max_len;  // context length the work plan was made for (rows before the append in a step)
  int32_t step;     // 1 in a fused decode step: full-width item 0 of each pair carries the append
  int32_t n_sink;
  int32_t window;
  int32_t slots;
  int32_t t_sl;
  int32_t t_mid;
  int32_t n_sl_items;
  int32_t sl_rows;
  int32_t items_per_b;
  int32_t partial_stride;
  int32_t combine_slices;  // channel slices per (pair, query head) in the combine (0: one wavefront each)
  float qk_scale;          // softmax scale * log2(e)
  // low-bit middle streams (segments in the canonical layout of leank_plan_layer_q)
  const uint8_t* k_q;
  const float* k_qp;
  const uint16_t* k_stage;
  const uint8_t* v_q;
  const float* v_qp;
  int64_t q_groups;  // K groups per (batch row, head): ceil(mid_cap / 64)
  int32_t n_batch;
  int32_t paged;     // middle rows in pages of LEANK_PAGE_ROWS through block_table
  // paged middle: page p of the pool starts at pool + p * page_elems; head
  // h's K rows at k_off, its V blocks at v_off within the page
  const uint16_t* pool;
  const int32_t* block_table;  // [batch][pages_per_row]
  int64_t page_elems;
  int32_t pages_per_row;
  int32_t pad_p;
  DecodeHead heads[LEANK_MAX_KV_HEADS];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load of streamed cache data (read once per call).
__device__ __forceinline__ u32x4_t load_stream16(const uint16_t* p) {
#if LEANK_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#else
  return *reinterpret_cast<const u32x4_t*>(p);
#endif
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// max / sum over the 16 lanes of a row, result in every lane of the row
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f32<kDppRowMirror>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  return x + dpp_f32<kDppRowMirror>(x);
}

// Per-wavefront running state.  Register i of lane l belongs to query head
// 4 * (l / 16) + i of the group; o[n] holds channels 16 n + l % 16.
struct WaveState {
  f32x4_t o[8];  // weighted V
  float m[4];    // reference max of the head (uniform over the 16-lane row)
  float l[4];    // this lane's part of the head's weight sum
};

// K and V operands of one 32-row tile.
template <int KB>
struct TileRegs {
  u32x4_t kf[2][KB];  // K rows t0 + 16 j + col, channels 32 kk + 8 grp .. +7
  u32x4_t vf[8];      // V block t0 / 8 + grp, channel 16 n + col
};

// Issues the loads of the tile starting at row t0 (rows >= nvalid are
// outside the item).  kb: K row 0 (row length kstride = c elements); vb: V
// block 0 of the stream.
template <int KB>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ kb, int kstride,
                                          const uint16_t* __restrict__ vb, int t0, int nvalid,
                                          int c, TileRegs<KB>& tr) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const uint16_t* kt = kb + static_cast<int64_t>(t0) * kstride;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const int row = 16 * j + col;
      const int ch = 32 * kk + 8 * grp;
      const bool ok = ch < c && row < nvalid;
      tr.kf[j][kk] = ok ? load_stream16(kt + row * kstride + ch) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const uint16_t* vt = vb + (static_cast<int64_t>(t0 / 8 + grp) * LEANK_HEAD_DIM + col) * 8;
  const bool v_ok = 8 * grp < nvalid;
#pragma unroll
  for (int n = 0; n < 8; ++n)
    tr.vf[n] = v_ok ? load_stream16(vt + n * 16 * 8) : u32x4_t{0u, 0u, 0u, 0u};
}

// Scores, softmax bookkeeping and weighted V of one loaded tile.  The
// masked variant (kTail) drops rows >= nvalid and row excl_rel (a ring row
// that a fused step replaces; any value outside [0, 32) drops nothing).
template <int G, int KB, bool kTail>
__device__ __forceinline__ void compute_tile(TileRegs<KB>& tr, int nvalid, int excl_rel,
                                             const u32x4_t (&qa)[KB],
                                             float qk_scale, uint16_t* __restrict__ p_lds,
                                             WaveState& st) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;

  // scores: s[j][i] = head 4 grp + i, row 16 j + col
  f32x4_t s[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    s[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) s[j] = mfma_bf16(qa[kk], tr.kf[j][kk], s[j]);
  }

  float mx[4];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v = s[j][i] * qk_scale;
      if (kTail && (16 * j + col >= nvalid || 16 * j + col == excl_rel)) v = -INFINITY;
      s[j][i] = v;
    }
    mx[i] = fmaxf(s[0][i], s[1][i]);  // this lane's rows
    grow |= mx[i] > st.m[i] + kRescaleSlack;
  }
  // a head's tile maximum passes its reference by more than the slack iff
  // one of its lanes does, so the row reductions run only then
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float tile_max = row_max16(mx[i]);
      float corr = 1.0f;
      if (tile_max > st.m[i] + kRescaleSlack) {
        corr = st.m[i] == -INFINITY ? 0.0f : fast_exp2(st.m[i] - tile_max);
        st.m[i] = tile_max;
      }
      st.l[i] *= corr;
#pragma unroll
      for (int n = 0; n < 8; ++n) st.o[n][i] *= corr;
    }
  }

  // weights, staged in LDS as bf16 hi/lo parts: p_lds[part][head][row]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m_use = st.m[i] == -INFINITY ? 0.0f : st.m[i];
    const int head = 4 * grp + i;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float p = fast_exp2(s[j][i] - m_use);
      st.l[i] += p;
      // every head's row is written (rows of heads >= G only feed output
      // rows that are never recorded), so the stores need no branch
      const __bf16 hi = static_cast<__bf16>(p);
      const __bf16 lo = static_cast<__bf16>(p - static_cast<float>(hi));
      p_lds[head * kTileRows + 16 * j + col] = __builtin_bit_cast(uint16_t, hi);
      p_lds[(16 + head) * kTileRows + 16 * j + col] = __builtin_bit_cast(uint16_t, lo);
    }
  }
  const u32x4_t pa_hi = *reinterpret_cast<const u32x4_t*>(p_lds + col * kTileRows + 8 * grp);
  const u32x4_t pa_lo = *reinterpret_cast<const u32x4_t*>(p_lds + (16 + col) * kTileRows + 8 * grp);

  if (kTail) {
    // zero the V rows of the lane's block that are dropped
    u32x4_t keep;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e0 = 8 * grp + 2 * w, e1 = e0 + 1;
      keep[w] = (e0 < nvalid && e0 != excl_rel ? 0x0000ffffu : 0u) |
                (e1 < nvalid && e1 != excl_rel ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) tr.vf[n] &= keep;
  }

#pragma unroll
  for (int n = 0; n < 8; ++n) {
    st.o[n] = mfma_bf16(pa_hi, tr.vf[n], st.o[n]);
    st.o[n] = mfma_bf16(pa_lo, tr.vf[n], st.o[n]);
  }
}

// Rows [r0, r1) of one stream, except row excl (-1: none).
template <int G, int KB>
__device__ __forceinline__ void attend_range(const uint16_t* kb, int kstride, const uint16_t* vb,
                                             int r0, int r1, int excl, int c,
                                             const u32x4_t (&qa)[KB], float qk_scale,
                                             uint16_t* p_lds, WaveState& st) {
  const int wave = threadIdx.x >> 6;
  int t0 = r0 + wave * kTileRows;
#if LEANK_PREFETCH
  // the next tile's loads are in flight while this one computes
  TileRegs<KB> cur;
  if (t0 < r1) load_tile<KB>(kb, kstride, vb, t0, r1 - t0, c, cur);
  for (; t0 < r1; t0 += kWaves * kTileRows) {
    const int tn = t0 + kWaves * kTileRows;
    TileRegs<KB> nxt;
    if (tn < r1) load_tile<KB>(kb, kstride, vb, tn, r1 - tn, c, nxt);
    const int nvalid = r1 - t0;
    if (nvalid >= kTileRows && static_cast<unsigned>(excl - t0) >= kTileRows) {
      compute_tile<G, KB, false>(cur, kTileRows, -1, qa, qk_scale, p_lds, st);
    } else {
      compute_tile<G, KB, true>(cur, nvalid, excl - t0, qa, qk_scale, p_lds, st);
    }
    cur = nxt;
  }
#else
  for (; t0 < r1; t0 += kWaves * kTileRows) {
    const int nvalid = r1 - t0;
    TileRegs<KB> cur;
    load_tile<KB>(kb, kstride, vb, t0, nvalid, c, cur);
    if (nvalid >= kTileRows && static_cast<unsigned>(excl - t0) >= kTileRows) {
      compute_tile<G, KB, false>(cur, kTileRows, -1, qa, qk_scale, p_lds, st);
    } else {
      compute_tile<G, KB, true>(cur, nvalid, excl - t0, qa, qk_scale, p_lds, st);
    }
  }
#endif
}

// Middle rows [r0, r1) of a paged stream: r0 is a multiple of the page
// size and s_pages holds the physical pages of rows r0, r0 + 64, ...
// (tiles never straddle a page: both are 32-row aligned).
template <int G, int KB>
__device__ __forceinline__ void attend_range_paged(const uint16_t* pool, int64_t page_elems,
                                                   const int32_t* s_pages, int64_t k_off,
                                                   int64_t v_off, int r0, int r1, int c,
                                                   const u32x4_t (&qa)[KB], float qk_scale,
                                                   uint16_t* p_lds, WaveState& st) {
  const int wave = threadIdx.x >> 6;
  for (int t0 = r0 + wave * kTileRows; t0 < r1; t0 += kWaves * kTileRows) {
    const int nvalid = r1 - t0;
    const uint16_t* page = pool + static_cast<int64_t>(s_pages[(t0 - r0) / LEANK_PAGE_ROWS]) * page_elems;
    const int t_in = t0 % LEANK_PAGE_ROWS;
    TileRegs<KB> cur;
    load_tile<KB>(page + k_off, c, page + v_off, t_in, nvalid, c, cur);
    if (nvalid >= kTileRows) {
      compute_tile<G, KB, false>(cur, kTileRows, -1, qa, qk_scale, p_lds, st);
    } else {
      compute_tile<G, KB, true>(cur, nvalid, -1, qa, qk_scale, p_lds, st);
    }
  }
}

// ---------------------------------------------------------------- low-bit middle
//
// A middle item of a cache with low-bit streams reads, per 32-row tile:
//   K  codes of a complete 64-row group, fed to the score product as exact
//      bf16 integers (8-bit: the code; 4-bit: 128 + code through a byte
//      permute).  The group's per-channel scale is folded into the query
//      instead: with K = code * scale + min per channel,
//        q . K = sum_c (q_c scale_c) code_c + sum_c q_c min_c,
//      so each wavefront forms q_c * scale_c (bf16 hi + lo parts) and the
//      group's offset term once per group, and the per-element work of a
//      tile is only the code conversion.  In the group that is not complete
//      yet, the bf16 staging rows are read as they are;
//   V  codes of the 8-row blocks, turned into exact bf16 integers the same
//      way for the B operand of the PV product.  The per-token scale
//      multiplies the weight (p' = p * scale) and sum_t p_t * min'_t is
//      added to every channel of the head at the end (min' = min, or
//      min - 128 * scale for 4-bit codes).
// Each wavefront takes whole 64-row groups (items start on group
// boundaries), so a group's query operands serve its two tiles.

// Pointers of one (batch row, live head) pair's low-bit middle.
struct QSegment {
  const uint8_t* k_codes;  // row 0 of the pair's K codes
  const float* k_par;      // group 0 of the pair's (scale, min) pairs
  const uint16_t* k_stage; // the pair's staging rows
  const uint8_t* v_codes;  // block 0 of the pair's V codes
  const float* v_par;      // row 0 of the pair's (scale, min) pairs
  int full_rows;           // rows in complete groups for this call
};

template <int QB>
__device__ __forceinline__ QSegment q_segment(const DecodeParams& p, const DecodeHead& hd, int b,
                                              int t_mid) {
  const int64_t c = hd.kept;
  const int64_t batch_rows = p.n_batch;
  const int64_t g_rows = p.q_groups * LEANK_QUANT_GROUP;
  const int64_t v_blocks = p.v_mid_rows / LEANK_V_BLOCK;
  QSegment q;
  q.k_codes = p.k_q + (batch_rows * g_rows * hd.k_off + static_cast<int64_t>(b) * g_rows * c) * QB / 8;
  q.k_par = p.k_qp + (batch_rows * p.q_groups * hd.k_off + static_cast<int64_t>(b) * p.q_groups * c) * 2;
  q.k_stage = p.k_stage + batch_rows * LEANK_QUANT_GROUP * hd.k_off +
              static_cast<int64_t>(b) * LEANK_QUANT_GROUP * c;
  q.v_codes = p.v_q + (hd.v_off * batch_rows * v_blocks + static_cast<int64_t>(b) * v_blocks) *
                          (LEANK_HEAD_DIM * LEANK_V_BLOCK * QB / 8);
  q.v_par = p.v_qp + (hd.v_off * batch_rows * p.mid_cap + static_cast<int64_t>(b) * p.mid_cap) * 2;
  q.full_rows = t_mid / LEANK_QUANT_GROUP * LEANK_QUANT_GROUP;
  return q;
}

// Raw operands of one low-bit tile.  kStaged: the tile lies in the K group
// that is not complete yet, whose rows are read as staged (bf16).  The
// score product's column col of sub-tile j is row 2 col + j of the tile, so
// a lane holds the weights of two adjacent rows and stages them as one pair.
template <int KB, int QB, bool kStaged>
struct QTileRegs {
  u32x4_t kf[kStaged ? 2 : 1][kStaged ? KB : 1];     // staged K rows (bf16)
  uint32_t kc[2][kStaged ? 1 : KB][QB == 8 ? 2 : 1];  // K codes, 8 channels
  uint32_t vc[8][QB == 8 ? 2 : 1];                   // V codes, 8 rows of one channel
  float vs[2], vm[2];                                // (scale, min) of rows 2 col + j
};

template <int KB, int QB, bool kStaged>
__device__ __forceinline__ void load_tile_q(const QSegment& q, int c, int t0, int nvalid,
                                            QTileRegs<KB, QB, kStaged>& tr) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const int row = t0 + 2 * col + j;
      const int ch = 32 * kk + 8 * grp;
      const bool ok = ch < c && 2 * col + j < nvalid;
      if constexpr (kStaged) {
        tr.kf[j][kk] = ok ? load_stream16(q.k_stage + static_cast<int64_t>(row - q.full_rows) * c + ch)
                          : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        const uint8_t* src = q.k_codes + (static_cast<int64_t>(row) * c + ch) * QB / 8;
        if constexpr (QB == 8) {
          const uint2 w = ok ? *reinterpret_cast<const uint2*>(src) : make_uint2(0u, 0u);
          tr.kc[j][kk][0] = w.x;
          tr.kc[j][kk][QB == 8 ? 1 : 0] = w.y;
        } else {
          tr.kc[j][kk][0] = ok ? *reinterpret_cast<const uint32_t*>(src) : 0u;
        }
      }
    }
  }
  const bool v_ok = 8 * grp < nvalid;
  const uint8_t* vt = q.v_codes + (static_cast<int64_t>(t0 / 8 + grp) * LEANK_HEAD_DIM + col) *
                                      (LEANK_V_BLOCK * QB / 8);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const uint8_t* src = vt + n * 16 * (LEANK_V_BLOCK * QB / 8);
    if constexpr (QB == 8) {
      const uint2 w = v_ok ? *reinterpret_cast<const uint2*>(src) : make_uint2(0u, 0u);
      tr.vc[n][0] = w.x;
      tr.vc[n][QB == 8 ? 1 : 0] = w.y;
    } else {
      tr.vc[n][0] = v_ok ? *reinterpret_cast<const uint32_t*>(src) : 0u;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool ok = 2 * col + j < nvalid;
    const float2 pr = ok ? *reinterpret_cast<const float2*>(q.v_par + static_cast<int64_t>(t0 + 2 * col + j) * 2)
                         : make_float2(0.0f, 0.0f);
    tr.vs[j] = pr.x;
    tr.vm[j] = pr.y;
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// (a, b) rounded to bf16 (nearest even), a in the low half: one conversion
// instruction for the pair
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// (a, b) as bf16 pairs hi + lo with hi = bf16(x) and lo = bf16(x - hi): the
// sum keeps about 16 significant bits of each value
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// two floats that bf16 holds exactly (small integers), packed without
// rounding: the upper halves of their bit patterns
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// code e (0..7) of 8 packed codes
template <int QB>
__device__ __forceinline__ float code_f32(const uint32_t (&w)[QB == 8 ? 2 : 1], int e) {
  if (QB == 8) return static_cast<float>((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
  return static_cast<float>((w[0] >> (4 * e)) & 0xfu);
}

// Operand of 8 packed codes as exact bf16 integers, in the order of the
// 4-byte word(s) w: 8-bit codes in byte order; 4-bit codes as 128 + code,
// the low nibbles of bytes 0..3 then their high nibbles (one byte permute
// per pair against the exponent byte of 128).  A V block word (byte k: rows
// k and k + 4) thus gives rows 0..7 in order; a K code word (byte k:
// channels 2k and 2k + 1) gives channels 0, 2, 4, 6, 1, 3, 5, 7.
template <int QB>
__device__ __forceinline__ u32x4_t v_codes_bf16(const uint32_t (&w)[QB == 8 ? 2 : 1]) {
  u32x4_t r;
  if (QB == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = pack_exact_bf16x2(code_f32<QB>(w, 2 * k), code_f32<QB>(w, 2 * k + 1));
  } else {
    const uint32_t lo = w[0] & 0x0f0f0f0fu;          // low nibbles of bytes 0..3
    const uint32_t hi = (w[0] >> 4) & 0x0f0f0f0fu;   // high nibbles
    const uint32_t exp128 = 0x43434343u;             // high byte of bf16 128
    // bytes [code a, 0x43, code b, 0x43]: selectors 0-3 pick the codes, 4 the exponent
    r[0] = __builtin_amdgcn_perm(exp128, lo, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(exp128, lo, 0x04030402u);
    r[2] = __builtin_amdgcn_perm(exp128, hi, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(exp128, hi, 0x04030402u);
  }
  return r;
}

// Query operands of one complete K group for this lane (query head col,
// channels 32 kk + 8 grp .. +7): q_c * scale_c as bf16 hi + lo parts in the
// channel order of the lane's K code operand, and the group's offset term
// sum_c q_c min'_c of query head 4 grp + i in register i (the same for
// every row; min' = min - 128 * scale for 4-bit codes fed as 128 + code).
// Both carry the softmax scale, so the scores come out scaled.
template <int KB>
struct QGroupOps {
  u32x4_t qh[KB], ql[KB];
  f32x4_t bias;
};

// (scale, min) pairs of the lane's channels 32 kk + 8 grp .. +7 in group g
// (kept counts are multiples of 8, so the 8 channels are all kept or all not)
template <int KB>
__device__ __forceinline__ void load_group_par(const QSegment& q, int c, int g, f32x4_t (&par)[KB][4]) {
  const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) {
    const int ch = 32 * kk + 8 * grp;
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(q.k_par + (static_cast<int64_t>(g) * c + ch) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) par[kk][i] = ch < c ? src[i] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
}

template <int KB, int QB>
__device__ __forceinline__ void group_ops(const f32x4_t (&par)[KB][4], const u32x4_t (&qa)[KB],
                                          float qk_scale, QGroupOps<KB>& go) {
  go.bias = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) {
    float sc[8], mn[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[2 * i] = par[kk][i][0];
      mn[2 * i] = par[kk][i][1];
      sc[2 * i + 1] = par[kk][i][2];
      mn[2 * i + 1] = par[kk][i][3];
    }
    // the offset term: B operand = min' of the lane's channels (every row alike)
    u32x4_t mh, ml;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = QB == 4 ? fmaf(-128.0f, sc[2 * w], mn[2 * w]) : mn[2 * w];
      const float b = QB == 4 ? fmaf(-128.0f, sc[2 * w + 1], mn[2 * w + 1]) : mn[2 * w + 1];
      uint32_t hi, lo;
      split_bf16x2(a, b, hi, lo);
      mh[w] = hi;
      ml[w] = lo;
    }
    go.bias = mfma_bf16(qa[kk], mh, go.bias);
    go.bias = mfma_bf16(qa[kk], ml, go.bias);
    // scaled query in the code operand's channel order
    float qf[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      qf[2 * w] = __uint_as_float(qa[kk][w] << 16);
      qf[2 * w + 1] = __uint_as_float(qa[kk][w] & 0xffff0000u);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // 4-bit pairs: (0, 2), (4, 6), (1, 3), (5, 7)
      const int e0 = QB == 4 ? (w < 2 ? 4 * w : 4 * w - 7) : 2 * w;
      const int e1 = QB == 4 ? e0 + 2 : 2 * w + 1;
      uint32_t hi, lo;
      split_bf16x2(qf[e0] * sc[e0] * qk_scale, qf[e1] * sc[e1] * qk_scale, hi, lo);
      go.qh[kk][w] = hi;
      go.ql[kk][w] = lo;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) go.bias[i] *= qk_scale;
}

// Scores of one tile of a complete group, already times the softmax scale.
template <int KB, int QB>
__device__ __forceinline__ void group_scores(const QTileRegs<KB, QB, false>& tr,
                                             const QGroupOps<KB>& go, f32x4_t (&s)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    s[j] = go.bias;
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const u32x4_t kb = v_codes_bf16<QB>(tr.kc[j][kk]);
      s[j] = mfma_bf16(go.qh[kk], kb, s[j]);
      s[j] = mfma_bf16(go.ql[kk], kb, s[j]);
    }
  }
}

// Softmax update and PV product of one low-bit tile from its scores
// (s[j][i]: head 4 grp + i, row 2 col + j; raw dot products, or already
// times the softmax scale when kScaled).
template <int G, int QB, bool kTail, bool kScaled>
__device__ __forceinline__ void softmax_pv_q(f32x4_t (&s)[2], const uint32_t (&vc)[8][QB == 8 ? 2 : 1],
                                             const float (&vs)[2], const float (&vm)[2], int nvalid,
                                             float qk_scale, uint16_t* __restrict__ p_lds,
                                             WaveState& st, float (&vmin)[4]) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;

  float mx[4];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v = kScaled ? s[j][i] : s[j][i] * qk_scale;
      if (kTail && 2 * col + j >= nvalid) v = -INFINITY;
      s[j][i] = v;
    }
    mx[i] = fmaxf(s[0][i], s[1][i]);  // this lane's rows
    grow |= mx[i] > st.m[i] + kRescaleSlack;
  }
  // a head's tile maximum passes its reference by more than the slack iff
  // one of its lanes does, so the row reductions run only then
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float tile_max = row_max16(mx[i]);
      float corr = 1.0f;
      if (tile_max > st.m[i] + kRescaleSlack) {
        corr = st.m[i] == -INFINITY ? 0.0f : fast_exp2(st.m[i] - tile_max);
        st.m[i] = tile_max;
      }
      st.l[i] *= corr;
      vmin[i] *= corr;
#pragma unroll
      for (int n = 0; n < 8; ++n) st.o[n][i] *= corr;
    }
  }

  // per-token V scale folded into the weights; the minimum summed apart
  float vmin_row[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) vmin_row[j] = QB == 4 ? fmaf(-128.0f, vs[j], vm[j]) : vm[j];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m_use = st.m[i] == -INFINITY ? 0.0f : st.m[i];
    const int head = 4 * grp + i;
    float pv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float pw = fast_exp2(s[j][i] - m_use);  // 0 for a dropped row
      st.l[i] += pw;
      const bool valid = !kTail || 2 * col + j < nvalid;
      vmin[i] = valid ? fmaf(pw, vmin_row[j], vmin[i]) : vmin[i];
      pv[j] = valid ? pw * vs[j] : 0.0f;
    }
    // rows 2 col, 2 col + 1 as one hi and one lo pair; every head's row is
    // written (rows of heads >= G only feed output rows that are never
    // recorded), so the stores need no branch
    uint32_t hi, lo;
    split_bf16x2(pv[0], pv[1], hi, lo);
    reinterpret_cast<uint32_t*>(p_lds)[(head * kTileRows) / 2 + col] = hi;
    reinterpret_cast<uint32_t*>(p_lds)[((16 + head) * kTileRows) / 2 + col] = lo;
  }
  const u32x4_t pa_hi = *reinterpret_cast<const u32x4_t*>(p_lds + col * kTileRows + 8 * grp);
  const u32x4_t pa_lo = *reinterpret_cast<const u32x4_t*>(p_lds + (16 + col) * kTileRows + 8 * grp);

#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const u32x4_t vb = v_codes_bf16<QB>(vc[n]);
    st.o[n] = mfma_bf16(pa_hi, vb, st.o[n]);
    st.o[n] = mfma_bf16(pa_lo, vb, st.o[n]);
  }
}

// Middle rows [r0, r1) of a low-bit stream (r0 on a group boundary).
template <int G, int KB, int QB>
__device__ __forceinline__ void attend_range_q(const QSegment& q, int r0, int r1, int c,
                                               const u32x4_t (&qa)[KB], float qk_scale,
                                               uint16_t* p_lds, WaveState& st, float (&vmin)[4]) {
  const int wave = threadIdx.x >> 6;
  for (int g0 = r0 + wave * LEANK_QUANT_GROUP; g0 < r1; g0 += kWaves * LEANK_QUANT_GROUP) {
    if (g0 >= q.full_rows) {
      // the open group: staged bf16 rows, the last tile possibly partial
      for (int t0 = g0; t0 < r1 && t0 < g0 + LEANK_QUANT_GROUP; t0 += kTileRows) {
        const int nvalid = r1 - t0;
        QTileRegs<KB, QB, true> cur;
        load_tile_q<KB, QB, true>(q, c, t0, nvalid, cur);
        f32x4_t s[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) s[j] = mfma_bf16(qa[kk], cur.kf[j][kk], s[j]);
        }
        if (nvalid >= kTileRows)
          softmax_pv_q<G, QB, false, false>(s, cur.vc, cur.vs, cur.vm, kTileRows, qk_scale, p_lds, st, vmin);
        else
          softmax_pv_q<G, QB, true, false>(s, cur.vc, cur.vs, cur.vm, nvalid, qk_scale, p_lds, st, vmin);
      }
    } else {
      // a complete group (g0 + 64 <= full_rows <= r1): two whole tiles,
      // whose loads are issued with the group's parameters (for up to 64
      // kept channels; wider heads load the second tile after the first
      // one's scores, to stay within the register budget)
      constexpr bool kBothFirst = KB <= 2;
      f32x4_t par[KB][4];
      load_group_par<KB>(q, c, g0 / LEANK_QUANT_GROUP, par);
      QTileRegs<KB, QB, false> t_a, t_b;
      load_tile_q<KB, QB, false>(q, c, g0, kTileRows, t_a);
      if (kBothFirst) load_tile_q<KB, QB, false>(q, c, g0 + kTileRows, kTileRows, t_b);
      QGroupOps<KB> go;
      group_ops<KB, QB>(par, qa, qk_scale, go);
      f32x4_t s[2];
      group_scores<KB, QB>(t_a, go, s);
      if (!kBothFirst) load_tile_q<KB, QB, false>(q, c, g0 + kTileRows, kTileRows, t_b);
      softmax_pv_q<G, QB, false, true>(s, t_a.vc, t_a.vs, t_a.vm, kTileRows, qk_scale, p_lds, st, vmin);
      group_scores<KB, QB>(t_b, go, s);
      softmax_pv_q<G, QB, false, true>(s, t_b.vc, t_b.vs, t_b.vm, kTileRows, qk_scale, p_lds, st, vmin);
    }
  }
}

// A operand of the score product for this lane: query head col of the
// group, kept channels 32 kk + 8 grp .. +7 (zero past c or for col >= G).
template <int G, int KB>
__device__ __forceinline__ void gather_q(const uint16_t* s_q, const int16_t* s_idx, bool dense,
                                         int c, u32x4_t (&qa)[KB]) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int j = 32 * kk + 8 * grp + 2 * w + half;
        uint32_t v = 0;
        if (col < G && j < c) {
          const int ch = dense ? j : (s_idx[j] & (LEANK_HEAD_DIM - 1));
          v = s_q[col * LEANK_HEAD_DIM + ch];
        }
        word |= v << (16 * half);
      }
      qa[kk][w] = word;
    }
  }
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// The append of a fused decode step for one (batch row, KV head) pair
// (LeanK page, section 3.1 item 2): the token at position pos goes to its
// sink or ring row (with no window, to the middle), and the token it pushes
// out of the window, ring row `slot`, moves its kept K channels and -- for
// a live head -- its V to the middle.  The regular items of the call
// cover the rows cached before the append, minus that ring row; the two
// tokens are scored by the pair's full-width item 0, which stages them in
// LDS before its tile loop and writes the append after it.  V rows are
// written as whole 8-row blocks (read in the prologue, one row replaced in
// LDS, written back with 16-byte stores): a single row of a block is 128
// scattered 2-byte pieces, which the memory system handles far more slowly
// than the 2 KiB block.
struct StepTokens {
  bool ok;        // the row takes part (its position lies in the plan)
  bool new_full;  // the new token is a sink or window row (full width)
  bool new_in;    // the new token is attended (not a middle token of a dead head)
  bool leave_in;  // a token leaves the window of a live head
  bool to_ring;   // the new token is written to a sink or ring row
  int pos;
  int slot;       // ring row of the new token (and of the leaving one)
  int mid_row;    // middle row written by the append, -1 for none
};

__device__ __forceinline__ StepTokens step_tokens(const DecodeParams& p, int b, bool live) {
  StepTokens st;
  const int64_t pos = p.row_pos ? p.row_pos[b] : p.step_pos;
  st.ok = pos >= 0 && pos <= p.max_len;
  st.pos = st.ok ? static_cast<int>(pos) : 0;
  const int S = p.n_sink, W = p.window;
  st.new_full = st.pos < S || W > 0;
  st.new_in = st.ok && (st.new_full || live);
  st.leave_in = st.ok && live && W > 0 && st.pos - W >= S;
  st.to_ring = st.ok && st.new_full;
  st.slot = st.pos < S ? st.pos : (W > 0 ? S + (st.pos - S) % W : 0);
  st.mid_row = st.leave_in ? st.pos - W - S : (st.ok && live && !st.new_full ? st.pos - S : -1);
  return st;
}

// Element offsets of middle row r of head hd in batch row b: its K row and
// the V block that holds it (bf16 middle, paged or not).
__device__ __forceinline__ void middle_row_at(const DecodeParams& p, const DecodeHead& hd, int b,
                                              int64_t r, const uint16_t** k_row,
                                              const uint16_t** v_block) {
  if (p.paged) {
    const int64_t page = p.block_table[static_cast<int64_t>(b) * p.pages_per_row + r / LEANK_PAGE_ROWS];
    const uint16_t* base = p.pool + page * p.page_elems;
    const int64_t in = r % LEANK_PAGE_ROWS;
    *k_row = base + hd.k_off + in * hd.kept;
    *v_block = base + hd.v_off + (in / LEANK_V_BLOCK) * (LEANK_HEAD_DIM * LEANK_V_BLOCK);
  } else {
    *k_row = p.k_prun + hd.k_off + (static_cast<int64_t>(b) * p.mid_cap + r) * hd.kept;
    *v_block = p.v_mid + hd.v_off + static_cast<int64_t>(b) * p.v_mid_rows * LEANK_HEAD_DIM +
               (r / LEANK_V_BLOCK) * (LEANK_HEAD_DIM * LEANK_V_BLOCK);
  }
}

// Word `lane` of a token's compacted K row (kept channels 2 lane, 2 lane + 1
// of the head) from its full row in LDS.
__device__ __forceinline__ uint32_t compact_from_lds(const uint16_t* row, const int16_t* s_idx,
                                                     int kept, int lane) {
  const int j0 = 2 * lane;
  if (j0 >= kept) return 0u;
  return static_cast<uint32_t>(row[s_idx[j0] & (LEANK_HEAD_DIM - 1)]) |
         (static_cast<uint32_t>(row[s_idx[j0 + 1] & (LEANK_HEAD_DIM - 1)]) << 16);
}

// KBMAX: 32-channel blocks of the widest live head (low-bit streams only;
// 4 for bf16 caches).
template <int G, int QB, int KBMAX>
__global__ LEANK_SPLIT_ATTRS void decode_split_kernel(const DecodeParams p) {
  __shared__ float s_acc[kWaves][G][LEANK_HEAD_DIM];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ uint16_t s_q[G * LEANK_HEAD_DIM];
  __shared__ int16_t s_idx[LEANK_HEAD_DIM];
  __shared__ __attribute__((aligned(16))) uint16_t s_p[kWaves][2 * 16 * kTileRows];
  // fused step: K rows of the new token [0] and the leaving token [1], the
  // new token's V, the V blocks (8 rows, as stored) of the ring row [0] and
  // of the middle row [1] the append writes, and the two tokens' scaled
  // scores per query head (-inf when not attended)
  __shared__ __attribute__((aligned(16))) uint16_t s_tok_k[2][LEANK_HEAD_DIM];
  __shared__ __attribute__((aligned(16))) uint16_t s_tok_v[LEANK_HEAD_DIM];
  __shared__ __attribute__((aligned(16))) uint16_t s_vblk[2][LEANK_HEAD_DIM * LEANK_V_BLOCK];
  __shared__ float s_tok_s[2][G];
  // paged middle: the physical pages of the item's rows
  __shared__ int32_t s_pages[QB ? 1 : 64];
  // low-bit fused step: the middle token's V as the cache will hold it
  __shared__ float s_midv[QB ? LEANK_HEAD_DIM : 1];
  __shared__ float s_vpar[2];

  const int item = blockIdx.x;
  const int b = item / p.items_per_b;
  const int r = item - b * p.items_per_b;
  int h = 0;
  while (h + 1 < p.n_kv && r >= p.heads[h + 1].base) ++h;
  const DecodeHead hd = p.heads[h];
  const int local = r - hd.base;
  const bool middle = local >= p.n_sl_items;
  const bool carries_step = p.step && local == 0;  // block-uniform
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;

  // stage the group's q rows and the head's kept ids; clear the P staging
  const uint16_t* qh = p.q + (static_cast<int64_t>(b) * p.n_q + h * G) * LEANK_HEAD_DIM;
  if (t < G * 16)
    *reinterpret_cast<u32x4_t*>(s_q + t * 8) = *reinterpret_cast<const u32x4_t*>(qh + t * 8);
  if (QB == 0 && p.paged && middle && t >= 192) {
    // the item's pages (items span at most 64 pages: their rows are capped
    // by the plan's largest item size)
    const int first = (local - p.n_sl_items) * hd.mid_rows / LEANK_PAGE_ROWS;
    const int i = t - 192;
    if (i < hd.mid_rows / LEANK_PAGE_ROWS && first + i < p.pages_per_row)
      s_pages[i] = p.block_table[static_cast<int64_t>(b) * p.pages_per_row + first + i];
  }
  if ((middle || carries_step) && t >= 128 && t < 144)
    *reinterpret_cast<u32x4_t*>(s_idx + (t - 128) * 8) =
        *reinterpret_cast<const u32x4_t*>(p.kept_idx + h * LEANK_HEAD_DIM + (t - 128) * 8);
  for (int k = lane; k < 2 * 16 * kTileRows / 8; k += 64)
    reinterpret_cast<u32x4_t*>(s_p[wave])[k] = u32x4_t{0u, 0u, 0u, 0u};
  const int64_t pair = static_cast<int64_t>(b) * p.n_kv + h;
  StepTokens tok{};
  if (carries_step) {
    // the new token from k_new / v_new; the leaving one and the V blocks
    // the append rewrites from the cache
    tok = step_tokens(p, b, hd.kept > 0);
    const u32x4_t zero4{0u, 0u, 0u, 0u};
    if (t < 128) {
      // ring V block of the slot (16 bytes = one channel's 8 rows per thread)
      const uint16_t* blk = p.v_sl + pair * p.v_sl_rows * LEANK_HEAD_DIM +
                            static_cast<int64_t>(tok.slot / LEANK_V_BLOCK) * (LEANK_HEAD_DIM * LEANK_V_BLOCK);
      *reinterpret_cast<u32x4_t*>(s_vblk[0] + t * 8) =
          tok.to_ring || tok.leave_in ? *reinterpret_cast<const u32x4_t*>(blk + t * 8) : zero4;
    } else {
      // V_mid block of the middle row written
      const int c = t - 128;
      u32x4_t x = zero4;
      if (tok.mid_row >= 0) {
        if constexpr (QB != 0) {
          // the middle row's V code block (QB * 128 bytes)
          const QSegment qs = q_segment<QB>(p, hd, b, 0);
          constexpr int kBlkBytes = LEANK_HEAD_DIM * LEANK_V_BLOCK * QB / 8;
          if (c * 16 < kBlkBytes)
            x = *reinterpret_cast<const u32x4_t*>(qs.v_codes + static_cast<int64_t>(tok.mid_row / LEANK_V_BLOCK) * kBlkBytes + c * 16);
        } else {
          const uint16_t *k_row, *blk;
          middle_row_at(p, hd, b, tok.mid_row, &k_row, &blk);
          x = *reinterpret_cast<const u32x4_t*>(blk + c * 8);
        }
      }
      *reinterpret_cast<u32x4_t*>(s_vblk[1] + c * 8) = x;
      if (t >= 144 && t < 160) {
        const int c8 = (t - 144) * 8;
        *reinterpret_cast<u32x4_t*>(s_tok_k[0] + c8) =
            tok.ok ? *reinterpret_cast<const u32x4_t*>(p.k_new + pair * LEANK_HEAD_DIM + c8) : zero4;
      } else if (t >= 160 && t < 176) {
        const int c8 = (t - 160) * 8;
        *reinterpret_cast<u32x4_t*>(s_tok_v + c8) =
            tok.ok ? *reinterpret_cast<const u32x4_t*>(p.v_new + pair * LEANK_HEAD_DIM + c8) : zero4;
      } else if (t >= 176 && t < 192) {
        const int c8 = (t - 176) * 8;
        const uint16_t* ring_k = p.k_sl + (pair * p.slots + tok.slot) * LEANK_HEAD_DIM;
        *reinterpret_cast<u32x4_t*>(s_tok_k[1] + c8) =
            tok.leave_in ? *reinterpret_cast<const u32x4_t*>(ring_k + c8) : zero4;
      }
    }
  }
  __syncthreads();

  WaveState st;
  float vmin[4];  // low-bit middle: sum of weight * V row minimum, per head
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.m[i] = -INFINITY;
    st.l[i] = 0.0f;
    vmin[i] = 0.0f;
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) st.o[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint16_t* p_lds = s_p[wave];

  int t_sl = p.t_sl, t_mid = p.t_mid;
  int excl = -1;  // ring row replaced by a fused step's append
  if (p.step) {
    // rows cached before the append; the row of the token leaving the
    // window is scored by the step item
    const int64_t pos = p.row_pos ? p.row_pos[b] : p.step_pos;
    const bool ok = pos >= 0 && pos <= p.max_len;
    const int len = ok ? static_cast<int>(pos) : 0;
    if (ok && p.window > 0 && len - p.window >= p.n_sink)
      excl = p.n_sink + (len - p.n_sink) % p.window;
    t_sl = min(len, p.slots);
    t_mid = max(0, len - p.slots);
  } else if (p.ctx_lens) {  // ragged batch: this row may hold fewer tokens than the plan
    const int len = min(max(p.ctx_lens[b], 0), p.max_len);
    t_sl = min(len, p.slots);
    t_mid = max(0, len - p.slots);
  }
  if (!middle) {
    const int r0 = local * p.sl_rows;
    const int r1 = min(t_sl, r0 + p.sl_rows);
    const uint16_t* kb = p.k_sl + pair * p.slots * LEANK_HEAD_DIM;
    const uint16_t* vb = p.v_sl + pair * p.v_sl_rows * LEANK_HEAD_DIM;
    u32x4_t qa[4];
    gather_q<G, 4>(s_q, s_idx, true, LEANK_HEAD_DIM, qa);
    attend_range<G, 4>(kb, LEANK_HEAD_DIM, vb, r0, r1, excl, LEANK_HEAD_DIM, qa, p.qk_scale, p_lds,
                       st);
  } else {
    const int chunk_id = local - p.n_sl_items;
    const int r0 = chunk_id * hd.mid_rows;
    const int r1 = min(t_mid, r0 + hd.mid_rows);
    const int c = hd.kept;
    if constexpr (QB != 0) {
      const QSegment q = q_segment<QB>(p, hd, b, t_mid);
      const int kb = (c + 31) / 32;
      if (KBMAX == 1 || kb == 1) {
        u32x4_t qa[1];
        gather_q<G, 1>(s_q, s_idx, false, c, qa);
        attend_range_q<G, 1, QB>(q, r0, r1, c, qa, p.qk_scale, p_lds, st, vmin);
      } else if constexpr (KBMAX >= 2) {
        if (KBMAX == 2 || kb == 2) {
          u32x4_t qa[2];
          gather_q<G, 2>(s_q, s_idx, false, c, qa);
          attend_range_q<G, 2, QB>(q, r0, r1, c, qa, p.qk_scale, p_lds, st, vmin);
        } else if constexpr (KBMAX >= 3) {
          if (kb == 3) {
            u32x4_t qa[3];
            gather_q<G, 3>(s_q, s_idx, false, c, qa);
            attend_range_q<G, 3, QB>(q, r0, r1, c, qa, p.qk_scale, p_lds, st, vmin);
          } else {
            u32x4_t qa[4];
            gather_q<G, 4>(s_q, s_idx, false, c, qa);
            attend_range_q<G, 4, QB>(q, r0, r1, c, qa, p.qk_scale, p_lds, st, vmin);
          }
        }
      }
    } else if (p.paged) {
      switch ((c + 31) / 32) {
        case 1: {
          u32x4_t qa[1];
          gather_q<G, 1>(s_q, s_idx, false, c, qa);
          attend_range_paged<G, 1>(p.pool, p.page_elems, s_pages, hd.k_off, hd.v_off, r0, r1, c, qa,
                                   p.qk_scale, p_lds, st);
          break;
        }
        case 2: {
          u32x4_t qa[2];
          gather_q<G, 2>(s_q, s_idx, false, c, qa);
          attend_range_paged<G, 2>(p.pool, p.page_elems, s_pages, hd.k_off, hd.v_off, r0, r1, c, qa,
                                   p.qk_scale, p_lds, st);
          break;
        }
        case 3: {
          u32x4_t qa[3];
          gather_q<G, 3>(s_q, s_idx, false, c, qa);
          attend_range_paged<G, 3>(p.pool, p.page_elems, s_pages, hd.k_off, hd.v_off, r0, r1, c, qa,
                                   p.qk_scale, p_lds, st);
          break;
        }
        default: {
          u32x4_t qa[4];
          gather_q<G, 4>(s_q, s_idx, false, c, qa);
          attend_range_paged<G, 4>(p.pool, p.page_elems, s_pages, hd.k_off, hd.v_off, r0, r1, c, qa,
                                   p.qk_scale, p_lds, st);
          break;
        }
      }
    } else {
      const uint16_t* kb = p.k_prun + hd.k_off + static_cast<int64_t>(b) * p.mid_cap * c;
      const uint16_t* vb = p.v_mid + hd.v_off + static_cast<int64_t>(b) * p.v_mid_rows * LEANK_HEAD_DIM;
      switch ((c + 31) / 32) {
        case 1: {
          u32x4_t qa[1];
          gather_q<G, 1>(s_q, s_idx, false, c, qa);
          attend_range<G, 1>(kb, c, vb, r0, r1, -1, c, qa, p.qk_scale, p_lds, st);
          break;
        }
        case 2: {
          u32x4_t qa[2];
          gather_q<G, 2>(s_q, s_idx, false, c, qa);
          attend_range<G, 2>(kb, c, vb, r0, r1, -1, c, qa, p.qk_scale, p_lds, st);
          break;
        }
        case 3: {
          u32x4_t qa[3];
          gather_q<G, 3>(s_q, s_idx, false, c, qa);
          attend_range<G, 3>(kb, c, vb, r0, r1, -1, c, qa, p.qk_scale, p_lds, st);
          break;
        }
        default: {
          u32x4_t qa[4];
          gather_q<G, 4>(s_q, s_idx, false, c, qa);
          attend_range<G, 4>(kb, c, vb, r0, r1, -1, c, qa, p.qk_scale, p_lds, st);
          break;
        }
      }
    }
  }

  if constexpr (QB != 0) {
    if (carries_step && tok.mid_row >= 0) {  // block-uniform
      // the token that becomes middle row r, as the low-bit cache will hold
      // it: V quantized per token; K exact in staging (a step whose row
      // completes a K group is not fused: the host runs the append first)
      const int e = tok.mid_row % LEANK_V_BLOCK;
      if (wave == 0) {
        const int e_ring = tok.slot % LEANK_V_BLOCK;
        const float x0 = bf16_to_f32(tok.leave_in ? s_vblk[0][(2 * lane) * LEANK_V_BLOCK + e_ring] : s_tok_v[2 * lane]);
        const float x1 = bf16_to_f32(tok.leave_in ? s_vblk[0][(2 * lane + 1) * LEANK_V_BLOCK + e_ring]
                                                  : s_tok_v[2 * lane + 1]);
        uint32_t c0, c1;
        float sc, lo;
        quantize_v_row_regs(x0, x1, QB, &c0, &c1, &sc, &lo);
        s_midv[2 * lane] = fmaf(static_cast<float>(c0), sc, lo);
        s_midv[2 * lane + 1] = fmaf(static_cast<float>(c1), sc, lo);
        uint8_t* cb = reinterpret_cast<uint8_t*>(s_vblk[1]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int at = v_code_byte(2 * lane + u, e, QB);
          const uint32_t code = u ? c1 : c0;
          if (QB == 8) {
            cb[at] = static_cast<uint8_t>(code);
          } else {
            const int sh = v_code_shift(e);
            cb[at] = static_cast<uint8_t>((cb[at] & ~(0xF << sh)) | (code << sh));
          }
        }
        if (lane == 0) {
          s_vpar[0] = sc;
          s_vpar[1] = lo;
        }
      }
      __syncthreads();
    }
  }

  if (carries_step) {
    // scores of the two step tokens: full width for a sink / window row,
    // kept channels for a middle row (the leaving token, or the new one
    // when there is no window)
    for (int d = wave; d < 2 * G; d += kWaves) {
      const int g = d >> 1;
      const int which = d & 1;
      const bool full = which == 0 && tok.new_full;
      float part;
      if (full) {
        part = dot2_bf16(reinterpret_cast<const uint32_t*>(s_q)[g * 64 + lane],
                         reinterpret_cast<const uint32_t*>(s_tok_k[0])[lane], 0.0f);
      } else {
        part = dot2_bf16(compact_from_lds(s_q + g * LEANK_HEAD_DIM, s_idx, hd.kept, lane),
                         compact_from_lds(s_tok_k[which], s_idx, hd.kept, lane), 0.0f);
      }
      const float sum = wave_sum(part);
      const bool in = which == 0 ? tok.new_in : tok.leave_in;
      if (lane == 0) s_tok_s[which][g] = in ? sum * p.qk_scale : -INFINITY;
    }
  }

  // this wavefront's part of the record: heads 4 grp + i, channels 16 n + col
  const int col = lane & 15;
  const int grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l = row_sum16(st.l[i]);
    // low-bit middle: every channel of the head gets sum_t p_t * min'_t
    const float vm = QB != 0 ? row_sum16(vmin[i]) : 0.0f;
    const int head = 4 * grp + i;
    if (head < G) {
#pragma unroll
      for (int n = 0; n < 8; ++n) s_acc[wave][head][16 * n + col] = QB != 0 ? st.o[n][i] + vm : st.o[n][i];
      if (col == 0) {
        s_m[wave][head] = st.m[i];
        s_l[wave][head] = l;
      }
    }
  }
  __syncthreads();

  // one record per item: (acc[G][128], m[G], l[G]) merged over the
  // wavefronts (and, in a step, the two step tokens)
  float* rec = p.partials + static_cast<int64_t>(item) * p.partial_stride;
  for (int k = t; k < G * LEANK_HEAD_DIM; k += kThreads) {
    const int g = k / LEANK_HEAD_DIM;
    const int ch = k - g * LEANK_HEAD_DIM;
    float m = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_m[w][g]);
    float s_new = -INFINITY, s_leave = -INFINITY;
    if (carries_step) {
      s_new = s_tok_s[0][g];
      s_leave = s_tok_s[1][g];
      m = fmaxf(m, fmaxf(s_new, s_leave));
    }
    const float m_use = m == -INFINITY ? 0.0f : m;
    float a = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][g] - m_use);
      a = fmaf(s_acc[w][g][ch], f, a);
      l = fmaf(s_l[w][g], f, l);
    }
    if (carries_step) {
      // weights are 0 for a token not attended; its staged V is zero too
      const float w_new = fast_exp2(s_new - m_use);
      const float w_leave = fast_exp2(s_leave - m_use);
      const uint32_t v_leave =
          tok.leave_in ? s_vblk[0][ch * LEANK_V_BLOCK + tok.slot % LEANK_V_BLOCK] : 0u;
      float vn = __uint_as_float(static_cast<uint32_t>(s_tok_v[ch]) << 16);
      float vl = __uint_as_float(v_leave << 16);
      if constexpr (QB != 0) {
        // the middle token's V as the low-bit cache holds it
        if (tok.mid_row >= 0) (tok.leave_in ? vl : vn) = s_midv[ch];
      }
      a = fmaf(w_new, vn, a);
      a = fmaf(w_leave, vl, a);
      l += w_new + w_leave;
    }
    rec[k] = a;
    if (ch == 0) {
      rec[G * LEANK_HEAD_DIM + g] = m;
      rec[G * LEANK_HEAD_DIM + G + g] = l;
    }
  }

  if (carries_step && tok.ok && wave == 0) {
    // the append; this workgroup's reads of the ring row ended before the
    // merge, and no other item of the call uses the rows written here.
    // Lane `lane` owns channels 2 lane, 2 lane + 1: their K words and the
    // 16-byte groups of the two V blocks, so no lane reads another's LDS.
    const int e_ring = tok.slot % LEANK_V_BLOCK;
    const int e_mid = tok.mid_row % LEANK_V_BLOCK;
    if constexpr (QB != 0) {
      if (tok.mid_row >= 0) {
        // staged K row, V codes, V parameters
        const QSegment qs = q_segment<QB>(p, hd, b, 0);
        const int r = tok.mid_row;
        const int which = tok.leave_in ? 1 : 0;
        if (2 * lane < hd.kept)
          reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(qs.k_stage) +
                                      static_cast<int64_t>(r % LEANK_QUANT_GROUP) * hd.kept)[lane] =
              compact_from_lds(s_tok_k[which], s_idx, hd.kept, lane);
        constexpr int kBlkBytes = LEANK_HEAD_DIM * LEANK_V_BLOCK * QB / 8;
        if (lane < kBlkBytes / 16)
          reinterpret_cast<u32x4_t*>(const_cast<uint8_t*>(qs.v_codes) +
                                     static_cast<int64_t>(r / LEANK_V_BLOCK) * kBlkBytes)[lane] =
              reinterpret_cast<const u32x4_t*>(s_vblk[1])[lane];
        if (lane == 0)
          *reinterpret_cast<float2*>(const_cast<float*>(qs.v_par) + static_cast<int64_t>(r) * 2) =
              make_float2(s_vpar[0], s_vpar[1]);
      }
    } else if (tok.mid_row >= 0) {
      // middle row: kept K channels (compacted) and V
      const int which = tok.leave_in ? 1 : 0;
      const uint16_t *k_row_c, *blk_c;
      middle_row_at(p, hd, b, tok.mid_row, &k_row_c, &blk_c);
      if (2 * lane < hd.kept)
        reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(k_row_c))[lane] =
            compact_from_lds(s_tok_k[which], s_idx, hd.kept, lane);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ch = 2 * lane + u;
        s_vblk[1][ch * LEANK_V_BLOCK + e_mid] =
            tok.leave_in ? s_vblk[0][ch * LEANK_V_BLOCK + e_ring] : s_tok_v[ch];
      }
      uint16_t* blk = const_cast<uint16_t*>(blk_c);
      reinterpret_cast<u32x4_t*>(blk)[2 * lane] = reinterpret_cast<const u32x4_t*>(s_vblk[1])[2 * lane];
      reinterpret_cast<u32x4_t*>(blk)[2 * lane + 1] =
          reinterpret_cast<const u32x4_t*>(s_vblk[1])[2 * lane + 1];
    }
    if (tok.to_ring) {
      uint16_t* ring_k = const_cast<uint16_t*>(p.k_sl) + pair * p.slots * LEANK_HEAD_DIM;
      reinterpret_cast<uint32_t*>(ring_k)[tok.slot * 64 + lane] =
          reinterpret_cast<const uint32_t*>(s_tok_k[0])[lane];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ch = 2 * lane + u;
        s_vblk[0][ch * LEANK_V_BLOCK + e_ring] = s_tok_v[ch];
      }
      uint16_t* blk = const_cast<uint16_t*>(p.v_sl) + pair * p.v_sl_rows * LEANK_HEAD_DIM +
                      static_cast<int64_t>(tok.slot / LEANK_V_BLOCK) * (LEANK_HEAD_DIM * LEANK_V_BLOCK);
      reinterpret_cast<u32x4_t*>(blk)[2 * lane] = reinterpret_cast<const u32x4_t*>(s_vblk[0])[2 * lane];
      reinterpret_cast<u32x4_t*>(blk)[2 * lane + 1] =
          reinterpret_cast<const u32x4_t*>(s_vblk[0])[2 * lane + 1];
    }
  }
}

// Merges the records of one (batch row, KV head) pair for one query head g
// with one wavefront, for pairs of at most 64 items (used up to 16): lane i holds item i's
// maximum and weight sum, the wavefront reduces them, then every lane sums
// its two channels over the items in item order (loads issued four items
// ahead), so no LDS or barrier is involved.  Grid: pairs x G / 4 workgroups
// of 4 wavefronts.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_combine_wave_kernel(const DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int64_t pair = unit / G;
  const int g = static_cast<int>(unit - pair * G);
  if (pair >= static_cast<int64_t>(p.n_batch) * p.n_kv) return;  // whole wavefront
  const int b = static_cast<int>(pair / p.n_kv);
  const int h = static_cast<int>(pair - static_cast<int64_t>(b) * p.n_kv);
  const DecodeHead hd = p.heads[h];
  const int n_items = p.n_sl_items + hd.n_mid;
  const int64_t stride = p.partial_stride;
  const float* first = p.partials + (static_cast<int64_t>(b) * p.items_per_b + hd.base) * stride;
  const int m_off = G * LEANK_HEAD_DIM + g;
  const int l_off = G * LEANK_HEAD_DIM + G + g;

  const float m_i = lane < n_items ? first[lane * stride + m_off] : -INFINITY;
  const float l_i = lane < n_items ? first[lane * stride + l_off] : 0.0f;
  float m_all = m_i;
  for (int off = 32; off > 0; off >>= 1) m_all = fmaxf(m_all, __shfl_xor(m_all, off));
  const float m_use = m_all == -INFINITY ? 0.0f : m_all;
  const float w_i = lane < n_items ? fast_exp2(m_i - m_use) : 0.0f;
  const float total = wave_sum(w_i * l_i);

  const float* acc = first + g * LEANK_HEAD_DIM + 2 * lane;
  float2 a = make_float2(0.0f, 0.0f);
  int n = 0;
  for (; n + 4 <= n_items; n += 4) {
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float2*>(acc + (n + u) * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = __shfl(w_i, n + u);
      a.x = fmaf(v[u].x, w, a.x);
      a.y = fmaf(v[u].y, w, a.y);
    }
  }
  for (; n < n_items; ++n) {
    const float2 v = *reinterpret_cast<const float2*>(acc + n * stride);
    const float w = __shfl(w_i, n);
    a.x = fmaf(v.x, w, a.x);
    a.y = fmaf(v.y, w, a.y);
  }
  const float inv = total > 0.0f ? 1.0f / total : 0.0f;  // an empty row gives zeros
  float* out = p.out + (static_cast<int64_t>(b) * p.n_q + h * G + g) * LEANK_HEAD_DIM + 2 * lane;
  *reinterpret_cast<float2*>(out) = make_float2(a.x * inv, a.y * inv);
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
    const float inv = total > 0.0f ? 1.0f / total : 0.0f;  // an empty row gives zeros
    float* out = p.out + (static_cast<int64_t>(b) * p.n_q + h * G) * LEANK_HEAD_DIM + ch;
    *reinterpret_cast<float4*>(out) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

// Launches the split and combine kernels for G query heads per KV head.
// kb_max: 32-channel blocks of the widest live head.
template <int G, int QB>
int launch_decode(const DecodeParams& p, int64_t n_items, int64_t n_pairs, int kb_max,
                  hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(n_items));
  if constexpr (QB == 0) {
    (void)kb_max;
    hipLaunchKernelGGL((decode_split_kernel<G, 0, 4>), grid, dim3(kThreads), 0, s, p);
  } else if (kb_max > 2) {
    hipLaunchKernelGGL((decode_split_kernel<G, QB, 4>), grid, dim3(kThreads), 0, s, p);
  } else if (kb_max == 2) {
    hipLaunchKernelGGL((decode_split_kernel<G, QB, 2>), grid, dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<G, QB, 1>), grid, dim3(kThreads), 0, s, p);
  }
  LEANK_HIP_TRY(hipGetLastError());
  if (p.combine_slices == 0) {  // every pair has at most 64 items
    hipLaunchKernelGGL(decode_combine_wave_kernel<G>,
                       dim3(static_cast<unsigned>((n_pairs * G + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(decode_combine_kernel<G>,
                       dim3(static_cast<unsigned>(n_pairs * G * p.combine_slices)), dim3(kThreads),
                       0, s, p);
  }
  LEANK_HIP_TRY(hipGetLastError());
  return LEANK_OK;
}

}  // namespace leank
