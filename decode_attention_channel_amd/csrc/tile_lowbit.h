// Tiles of the low-bit middle streams (K codes per channel over 64-row
// groups, V codes per token).
#pragma once

#include "decode_base.h"

namespace leank {

// A paged low-bit middle holds one 64-row K group per page: the group
// number indexes the block table.
static_assert(LEANK_PAGE_ROWS == LEANK_QUANT_GROUP, "a page must hold exactly one K group");

// ---------------------------------------------------------------- low-bit middle
//
// A middle item of a cache with low-bit streams reads, per 64-row group
// (each wavefront takes whole groups; items start on group boundaries):
//   K  codes of a complete group, fed to the score product as exact bf16
//      integers (8-bit: the code; 4-bit: 128 + code through a byte
//      permute).  The group's per-channel scale is folded into the query
//      instead: with K = code * scale + min per channel,
//        q . K = sum_c (q_c scale_c) code_c + sum_c q_c min_c,
//      so each wavefront forms q_c * scale_c (bf16 hi + lo parts) and the
//      group's offset term once per group, and the per-element work is
//      only the code conversion.  The rows of the group that is not
//      complete yet are read from the bf16 staging rows as they are;
//   V  codes of the 8-row blocks, turned into exact bf16 integers the same
//      way for the B operand of the PV product.  The per-token scale
//      multiplies the weight (p' = p * scale) and sum_t p_t * min_t is
//      added to every channel of the head at the end; for 4-bit codes so is
//      -128 sum_t p'_t, with p'_t rounded as it entered the product, so the
//      offset cancels exactly.

// Pointers of one (batch row, live head) pair's low-bit middle: contiguous
// streams, or one page per 64-row group through the block table.
struct QSegment {
  const uint8_t* k_codes;  // row 0 of the pair's K codes (contiguous)
  const float* k_par;      // group 0 of the pair's (scale, min) pairs
  const uint16_t* k_stage; // the pair's staging rows
  const uint8_t* v_codes;  // block 0 of the pair's V codes
  const float* v_par;      // row 0 of the pair's (scale, min) pairs
  const uint8_t* pool;     // paged: the page pool, or null
  const int32_t* pages;    // paged: the row's block table entries
  int64_t page_bytes;
  int32_t pk_codes, pk_par, pv_codes, pv_par;  // paged: byte offsets within a page
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
  q.k_stage = p.k_stage + batch_rows * LEANK_QUANT_GROUP * hd.k_off +
              static_cast<int64_t>(b) * LEANK_QUANT_GROUP * c;
  q.full_rows = t_mid / LEANK_QUANT_GROUP * LEANK_QUANT_GROUP;
  if (p.paged) {
    q.pool = reinterpret_cast<const uint8_t*>(p.pool);
    q.pages = p.block_table + static_cast<int64_t>(b) * p.pages_per_row;
    q.page_bytes = 2 * p.page_elems;
    q.pk_codes = hd.pq_k_codes;
    q.pk_par = hd.pq_k_par;
    q.pv_codes = hd.pq_v_codes;
    q.pv_par = hd.pq_v_par;
    q.k_codes = nullptr;
    q.k_par = nullptr;
    q.v_codes = nullptr;
    q.v_par = nullptr;
    return q;
  }
  q.pool = nullptr;
  q.k_codes = p.k_q + (batch_rows * g_rows * hd.k_off + static_cast<int64_t>(b) * g_rows * c) * QB / 8;
  q.k_par = p.k_qp + (batch_rows * p.q_groups * hd.k_off + static_cast<int64_t>(b) * p.q_groups * c) * 2;
  q.v_codes = p.v_q + (hd.v_off * batch_rows * v_blocks + static_cast<int64_t>(b) * v_blocks) *
                          (LEANK_HEAD_DIM * LEANK_V_BLOCK * QB / 8);
  q.v_par = p.v_qp + (hd.v_off * batch_rows * p.mid_cap + static_cast<int64_t>(b) * p.mid_cap) * 2;
  return q;
}

// Where group g (rows 64 g ..) of a pair lives: its K codes (row 0 of the
// group), K (scale, min) pairs, first V code block and first V row
// parameters.
struct QGroup {
  const uint8_t* k_codes;
  const float* k_par;
  const uint8_t* v_codes;
  const float* v_par;
};

// page: the group's physical page (paged streams; read by the caller, so
// that a loop can fetch it ahead of use).
template <int QB>
__device__ __forceinline__ QGroup q_group_at_page(const QSegment& q, int c, int g, int page) {
  QGroup a;
  if (q.pool) {
    const uint8_t* base = q.pool + static_cast<int64_t>(page) * q.page_bytes;
    a.k_codes = base + q.pk_codes;
    a.k_par = reinterpret_cast<const float*>(base + q.pk_par);
    a.v_codes = base + q.pv_codes;
    a.v_par = reinterpret_cast<const float*>(base + q.pv_par);
  } else {
    a.k_codes = q.k_codes + static_cast<int64_t>(g) * LEANK_QUANT_GROUP * c * QB / 8;
    a.k_par = q.k_par + static_cast<int64_t>(g) * c * 2;
    a.v_codes = q.v_codes + static_cast<int64_t>(g) * (LEANK_QUANT_GROUP / LEANK_V_BLOCK) *
                                (LEANK_HEAD_DIM * LEANK_V_BLOCK * QB / 8);
    a.v_par = q.v_par + static_cast<int64_t>(g) * LEANK_QUANT_GROUP * 2;
  }
  return a;
}

template <int QB>
__device__ __forceinline__ QGroup q_group(const QSegment& q, int c, int g) {
  return q_group_at_page<QB>(q, c, g, q.pool ? q.pages[g] : 0);
}

// Raw operands of one tile of the open K group (the group that is not
// complete yet, whose K rows are read as staged bf16).  The score
// product's column col of sub-tile j is row 2 col + j of the tile, so a
// lane holds the weights of two adjacent rows and stages them as one pair.
template <int KB, int QB>
struct QTileRegs {
  u32x4_t kf[2][KB];                 // staged K rows (bf16)
  uint32_t vc[8][QB == 8 ? 2 : 1];  // V codes, 8 rows of one channel
  float vs[2], vm[2];               // (scale, min) of rows 2 col + j
};

template <int KB, int QB>
__device__ __forceinline__ void load_tile_q(const QSegment& q, int c, int t0, int nvalid,
                                            QTileRegs<KB, QB>& tr) {
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
      tr.kf[j][kk] = ok ? load_stream16(q.k_stage + static_cast<int64_t>(row - q.full_rows) * c + ch)
                        : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const bool v_ok = 8 * grp < nvalid;
  const QGroup at = q_group<QB>(q, c, t0 / LEANK_QUANT_GROUP);
  const int t_in = t0 % LEANK_QUANT_GROUP;  // tiles never straddle a group
  const uint8_t* vt = at.v_codes + ((t_in / 8 + grp) * LEANK_HEAD_DIM + col) * (LEANK_V_BLOCK * QB / 8);
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
    const float2 pr = ok ? *reinterpret_cast<const float2*>(at.v_par + (t_in + 2 * col + j) * 2)
                         : make_float2(0.0f, 0.0f);
    tr.vs[j] = pr.x;
    tr.vm[j] = pr.y;
  }
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

// ---------------------------------------------------------------- complete groups
//
// The 64 rows of a complete K group are scored with v_mfma_f32_4x4x4_16b_bf16
// (16 blocks of 4 rows; lane l = 4 blk + j): row l of the group is lane l,
// whose B operand is 4 of its K codes as exact bf16 integers, and the A
// operand of lane l is 4 channels of q_c * scale_c for query head l % 4 of
// a quad of heads; register i of lane l comes out as the score of head
// 4 qd + i and row l.  Each lane thus holds every head's score of one row:
// the softmax bookkeeping runs once per (row, head) instead of once per
// (row, head slot of the 16 the 16x16 product has), and needs no
// reductions unless a reference maximum moves.  The channel order of a K
// code operand follows v_codes_bf16 (4-bit: the even channels of a 4-byte
// word, then the odd ones); the scaled query is laid out in the same order.
// The group's offset term sum_c q_c min'_c starts the accumulators.

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma4_bf16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Per-wavefront LDS of the group path, in 16-bit units: the weight staging
// [part 2][head 16][row 64] (4 KiB), then the group's (scale, min) pairs
// (4 c) and the scaled-query table, hi and lo parts [quad][4-channel
// step][head 4][4] (8 NQ c).  The staging rows of heads the group does not
// write keep finite values (zeros, or earlier weights).
constexpr int kGroupStage = 2 * 16 * 64;
template <int KBMAX, int G>
constexpr int group_lds_halves() {
  return kGroupStage + 4 * 32 * KBMAX + 8 * ((G + 3) / 4) * 32 * KBMAX;
}

// Softmax state of the group path: register i of quad qd is query head
// 4 qd + i; the reference maximum is uniform over the wavefront, the sums
// are this lane's (row's) parts.
template <int NQ>
struct RowState {
  float m[NQ][4];
  float l[NQ][4];
  float vmin[NQ][4];  // sum of weight * V row minimum'
};

// wavefront maximum
__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// Raw operands of one complete group for this lane: K codes of row lane
// (c * QB / 8 bytes), V codes of both 32-row halves, the row's V (scale, min).
template <int KB, int QB>
struct GroupRegs {
  f32x4_t par;           // 16 bytes of the group's (scale, min) pairs (used in lanes < c / 2)
  uint32_t kc[KB * QB];  // 4-byte words of the K code row (8 or 4 channels each)
  uint32_t vc[2][8][QB == 8 ? 2 : 1];
  float vs, vm;
};

// kBranchFree: every lane issues every load (past the data it reloads the
// first words, which are not used), so the loads take no branches and the
// compiler's waits for them stay exact in a software pipeline; otherwise
// words past the data are zeros.
// kPart: 0 every load of the group, 1 its K codes and parameters only, 2 its
// V codes only.
template <int KB, int QB, bool kBranchFree, int kPart = 0>
__device__ __forceinline__ void load_group(const QSegment& q, int c, int g0, int page,
                                           GroupRegs<KB, QB>& gr) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const QGroup at = q_group_at_page<QB>(q, c, g0 / LEANK_QUANT_GROUP, page);
  // the group's parameters first: the query tables wait only for them
  // (they use lanes 4 lane < 2 c)
  if constexpr (kPart != 2) {
  if constexpr (kBranchFree)
    gr.par = *reinterpret_cast<const f32x4_t*>(at.k_par + (4 * lane < 2 * c ? 4 * lane : 0));
  else
    gr.par = 4 * lane < 2 * c ? *reinterpret_cast<const f32x4_t*>(at.k_par + 4 * lane)
                              : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // the row's codes: c * QB / 8 bytes, a multiple of 4 (8-bit: of 8)
  const uint8_t* krow = at.k_codes + lane * c * QB / 8;
  if constexpr (QB == 8) {
#pragma unroll
    for (int i = 0; i < KB * QB / 2; ++i) {
      uint2 w;
      if constexpr (kBranchFree)
        w = *reinterpret_cast<const uint2*>(krow + (8 * i < c ? 8 * i : 0));
      else
        w = 8 * i < c ? *reinterpret_cast<const uint2*>(krow + 8 * i) : make_uint2(0u, 0u);
      gr.kc[2 * i] = w.x;
      gr.kc[2 * i + 1] = w.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KB * QB; ++i) {
      if constexpr (kBranchFree)
        gr.kc[i] = *reinterpret_cast<const uint32_t*>(krow + (8 * i < c ? 4 * i : 0));
      else
        gr.kc[i] = 8 * i < c ? *reinterpret_cast<const uint32_t*>(krow + 4 * i) : 0u;
    }
  }
  }
  if constexpr (kPart != 1) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint8_t* vt = at.v_codes + ((4 * half + grp) * LEANK_HEAD_DIM + col) * (LEANK_V_BLOCK * QB / 8);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint8_t* src = vt + n * 16 * (LEANK_V_BLOCK * QB / 8);
      if constexpr (QB == 8) {
        const uint2 w = *reinterpret_cast<const uint2*>(src);
        gr.vc[half][n][0] = w.x;
        gr.vc[half][n][QB == 8 ? 1 : 0] = w.y;
      } else {
        gr.vc[half][n][0] = *reinterpret_cast<const uint32_t*>(src);
      }
    }
  }
  }
  if constexpr (kPart != 2) {
    const float2 pr = *reinterpret_cast<const float2*>(at.v_par + lane * 2);
    gr.vs = pr.x;
    gr.vm = pr.y;
  }
}

// The table entries and offset terms of the complete groups are split over
// the lanes the same way in every group: lane l takes query head
// h = l / kLanes and kept channels j = l % kLanes + kLanes k.  QueryCols
// holds, per lane, q_h at those channels (0 for heads >= G or channels
// past c), gathered once per item: a group then only scales them.
// (Wide heads, more than 4 values per lane, keep the LDS pointers instead
// and gather in every group: holding the values spilled registers.)
template <int NQ>
constexpr int query_lanes() { return 64 / (NQ * 4); }  // lanes per head: 16 or 8
template <int KB, int NQ>
constexpr int query_cols() { return 32 * KB / query_lanes<NQ>(); }
template <int KB, int NQ>
constexpr bool kHoldQueryCols = query_cols<KB, NQ>() <= 4;
template <int KB, int NQ>
struct QueryCols {
  float qv[kHoldQueryCols<KB, NQ> ? query_cols<KB, NQ>() : 1];
  const uint16_t* s_q;
  const int16_t* s_idx;
  int h_limit;  // G
};

// q of this lane's head at kept channel j (0 past c or for heads >= G)
__device__ __forceinline__ float query_col(const uint16_t* s_q, const int16_t* s_idx, int h, int j,
                                           int c, int g) {
  return h < g && j < c ? bf16_to_f32(s_q[h * LEANK_HEAD_DIM + (s_idx[j] & (LEANK_HEAD_DIM - 1))]) : 0.0f;
}

template <int G, int KB, int NQ>
__device__ __forceinline__ void gather_query_cols(const uint16_t* s_q, const int16_t* s_idx, int c,
                                                  QueryCols<KB, NQ>& qc) {
  constexpr int kLanes = query_lanes<NQ>();
  const int lane = threadIdx.x & 63;
  const int h = lane / kLanes;
  const int part = lane - h * kLanes;
  qc.s_q = s_q;
  qc.s_idx = s_idx;
  qc.h_limit = G;
  if constexpr (kHoldQueryCols<KB, NQ>) {
#pragma unroll
    for (int k = 0; k < query_cols<KB, NQ>(); ++k) qc.qv[k] = query_col(s_q, s_idx, h, part + kLanes * k, c, G);
  }
}

// Builds the group's query tables in this wavefront's LDS and returns the
// offset term of quad qd's head i in bias[qd][i] (every lane): q' = q *
// scale * qk_scale (hi + lo); the offset is qk_scale sum_c q_c min_c, and
// for 4-bit codes also -128 sum_c q'_c (q'_c as rounded in the table).
template <int G, int NQ, int QB, int KB>
__device__ __forceinline__ void build_group_tables(const f32x4_t& par16, int c,
                                                   const QueryCols<KB, NQ>& qc, float qk_scale,
                                                   uint16_t* w_lds, float (&bias)[NQ][4]) {
  constexpr int kLanes = query_lanes<NQ>();
  const int lane = threadIdx.x & 63;
  float* par = reinterpret_cast<float*>(w_lds + kGroupStage);  // [c][2]
  uint16_t* tab = w_lds + kGroupStage + 4 * c;                // hi [NQ][c/4][4][4], then lo
  // the (scale, min) pairs, 16 bytes per lane, to LDS
  if (4 * lane < 2 * c) reinterpret_cast<f32x4_alias_t*>(par)[lane] = par16;
  // this lane's entries (head h, kept channel j), and its part of head h's
  // offset sum: sum_c q_c min_c (times the softmax scale), and for 4-bit
  // codes, which enter the product as 128 + code, -128 sum_c q'_c with
  // q'_c rounded as it entered the product (hi + lo), so that the 128
  // terms cancel.  Every head slot's entries are written (zeros for heads
  // >= G).
  const int h = lane / kLanes;
  const int part = lane - h * kLanes;
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < query_cols<KB, NQ>(); ++k) {
    const int j = part + kLanes * k;
    if (j < c) {
      const float2 pm = *reinterpret_cast<const float2*>(par + 2 * j);
      float qv;
      if constexpr (kHoldQueryCols<KB, NQ>)
        qv = qc.qv[k];
      else
        qv = query_col(qc.s_q, qc.s_idx, h, j, c, qc.h_limit);
      const float x = qv * pm.x * qk_scale;
      const __bf16 hi = static_cast<__bf16>(x);
      const __bf16 lo = static_cast<__bf16>(x - static_cast<float>(hi));
      // 4-channel step and place of channel j in the code operand order
      const int step = QB == 4 ? 2 * (j >> 3) + (j & 1) : j >> 2;
      const int pos = QB == 4 ? (j & 7) >> 1 : j & 3;
      const int at = (((h >> 2) * (c / 4) + step) * 4 + (h & 3)) * 4 + pos;
      tab[at] = __builtin_bit_cast(uint16_t, hi);
      tab[NQ * 4 * c + at] = __builtin_bit_cast(uint16_t, lo);
      if constexpr (QB == 4) {
        sum = fmaf(qv * qk_scale, pm.y, sum);
        sum = fmaf(-128.0f, static_cast<float>(hi) + static_cast<float>(lo), sum);
      } else {
        sum = fmaf(qv, pm.y, sum);
      }
    }
  }
  sum += dpp_f32<kDppQuadXor1>(sum);
  sum += dpp_f32<kDppQuadXor2>(sum);
  sum += dpp_f32<kDppHalfMirror>(sum);
  if (kLanes == 16) sum += dpp_f32<kDppRowMirror>(sum);
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bias[qd][i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), (4 * qd + i) * kLanes)) *
                    (QB == 4 ? 1.0f : qk_scale);
  }
}

// One complete group of 64 rows starting at g0 (group g0 / 64).
template <int G, int KB, int QB>
__device__ __forceinline__ void attend_group(const GroupRegs<KB, QB>& gr, int c,
                                             const QueryCols<KB, (G + 3) / 4>& qc, float qk_scale,
                                             uint16_t* w_lds, RowState<(G + 3) / 4>& rs,
                                             WaveState& st) {
  constexpr int NQ = (G + 3) / 4;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;

  float bias[NQ][4];
  build_group_tables<G, NQ, QB, KB>(gr.par, c, qc, qk_scale, w_lds, bias);

  // scores (already times the softmax scale)
  f32x4_t s[NQ];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) s[qd] = f32x4_t{bias[qd][0], bias[qd][1], bias[qd][2], bias[qd][3]};
  const uint16_t* tab = w_lds + kGroupStage + 4 * c;
#pragma unroll
  for (int w = 0; w < KB * QB; ++w) {  // 4-byte words of the row's codes
    if (4 * w >= c * QB / 8) continue;  // past the row (c < 32 KB)
    // code operands of the word: 4-bit: two 4-channel steps; 8-bit: one
    uint2 kb[QB == 4 ? 2 : 1];
    if constexpr (QB == 4) {
      const uint32_t wv = gr.kc[w];
      const uint32_t lo = wv & 0x0f0f0f0fu, hi = (wv >> 4) & 0x0f0f0f0fu;
      kb[0] = make_uint2(__builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u),
                         __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u));
      kb[QB == 4 ? 1 : 0] = make_uint2(__builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u),
                                       __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u));
    } else {
      const uint32_t wv = gr.kc[w];
      kb[0] = make_uint2(pack_exact_bf16x2(static_cast<float>(wv & 0xffu), static_cast<float>((wv >> 8) & 0xffu)),
                         pack_exact_bf16x2(static_cast<float>((wv >> 16) & 0xffu), static_cast<float>(wv >> 24)));
    }
#pragma unroll
    for (int u = 0; u < (QB == 4 ? 2 : 1); ++u) {
      const int step = (QB == 4 ? 2 : 1) * w + u;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        const int at = ((qd * (c / 4) + step) * 4 + (lane & 3)) * 4;
        const u32x2_alias_t ahv = *reinterpret_cast<const u32x2_alias_t*>(tab + at);
        const u32x2_alias_t alv = *reinterpret_cast<const u32x2_alias_t*>(tab + NQ * 4 * c + at);
        const uint2 ah = make_uint2(ahv[0], ahv[1]), al = make_uint2(alv[0], alv[1]);
        s[qd] = mfma4_bf16(ah, kb[u], s[qd]);
        s[qd] = mfma4_bf16(al, kb[u], s[qd]);
      }
    }
  }

  // the reference maxima move only when a score passes one by the slack
  bool grow = false;
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
    for (int i = 0; i < 4; ++i) grow |= s[qd][i] > rs.m[qd][i] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    float corr[NQ][4];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mx = wave_max(s[qd][i]);
        corr[qd][i] = 1.0f;
        if (mx > rs.m[qd][i] + kRescaleSlack) {
          corr[qd][i] = rs.m[qd][i] == -INFINITY ? 0.0f : fast_exp2(rs.m[qd][i] - mx);
          rs.m[qd][i] = mx;
        }
        rs.l[qd][i] *= corr[qd][i];
        rs.vmin[qd][i] *= corr[qd][i];
      }
    }
    // accumulator rows of head 4 grp + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f = 1.0f;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) f = grp == qd ? corr[qd][i] : f;
#pragma unroll
      for (int n = 0; n < 8; ++n) st.o[n][i] *= f;
    }
  }

  // weights, staged as bf16 hi / lo: w_lds[part][head][row].  4-bit codes
  // enter the product as 128 + code; the offset is taken out with the weight
  // as it enters the product (hi + lo), so that the two 128 terms cancel and
  // only the weight's rounding times the code (at most 15) remains
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m_use = rs.m[qd][i] == -INFINITY ? 0.0f : rs.m[qd][i];
      const float pw = fast_exp2(s[qd][i] - m_use);
      rs.l[qd][i] += pw;
      const float pv = pw * gr.vs;
      const __bf16 hi = static_cast<__bf16>(pv);
      const __bf16 lo = static_cast<__bf16>(pv - static_cast<float>(hi));
      const float in_product = static_cast<float>(hi) + static_cast<float>(lo);
      rs.vmin[qd][i] = QB == 4 ? fmaf(-128.0f, in_product, fmaf(pw, gr.vm, rs.vmin[qd][i]))
                               : fmaf(pw, gr.vm, rs.vmin[qd][i]);
      const int head = 4 * qd + i;
      if (head < G) {
        w_lds[head * 64 + lane] = __builtin_bit_cast(uint16_t, hi);
        w_lds[(16 + head) * 64 + lane] = __builtin_bit_cast(uint16_t, lo);
      }
    }
  }

  // P V over the two 32-row halves (A operand: head col, rows 8 grp .. +7)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const u32x4_t pa_hi = *reinterpret_cast<const u32x4_alias_t*>(w_lds + col * 64 + 32 * half + 8 * grp);
    const u32x4_t pa_lo = *reinterpret_cast<const u32x4_alias_t*>(w_lds + (16 + col) * 64 + 32 * half + 8 * grp);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const u32x4_t vb = v_codes_bf16<QB>(gr.vc[half][n]);
      st.o[n] = mfma_bf16(pa_hi, vb, st.o[n]);
      st.o[n] = mfma_bf16(pa_lo, vb, st.o[n]);
    }
  }
}

// Softmax update and PV product of one tile of the open group from its
// raw scores (s[j][i]: head 4 grp + i, row 2 col + j).
template <int G, int QB, bool kTail>
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
      float v = s[j][i] * qk_scale;
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
  // (for 4-bit codes, which enter the product as 128 + code, with the
  // offset taken out by the weight as it enters the product, hi + lo, so
  // that the 128 terms cancel)
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
      vmin[i] = valid ? fmaf(pw, vm[j], vmin[i]) : vmin[i];
      pv[j] = valid ? pw * vs[j] : 0.0f;
    }
    // rows 2 col, 2 col + 1 as one hi and one lo pair; every head's row is
    // written (rows of heads >= G only feed output rows that are never
    // recorded), so the stores need no branch
    uint32_t hi, lo;
    split_bf16x2(pv[0], pv[1], hi, lo);
    if constexpr (QB == 4) {
      const float in0 = __uint_as_float(hi << 16) + __uint_as_float(lo << 16);
      const float in1 = __uint_as_float(hi & 0xffff0000u) + __uint_as_float(lo & 0xffff0000u);
      vmin[i] = fmaf(-128.0f, in0 + in1, vmin[i]);
    }
    reinterpret_cast<uint32_t*>(p_lds)[(head * kTileRows) / 2 + col] = hi;
    reinterpret_cast<uint32_t*>(p_lds)[((16 + head) * kTileRows) / 2 + col] = lo;
  }
  const u32x4_t pa_hi = *reinterpret_cast<const u32x4_alias_t*>(p_lds + col * kTileRows + 8 * grp);
  const u32x4_t pa_lo = *reinterpret_cast<const u32x4_alias_t*>(p_lds + (16 + col) * kTileRows + 8 * grp);

#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const u32x4_t vb = v_codes_bf16<QB>(vc[n]);
    st.o[n] = mfma_bf16(pa_hi, vb, st.o[n]);
    st.o[n] = mfma_bf16(pa_lo, vb, st.o[n]);
  }
}

// Whether a wavefront loads its next complete group while it scores the
// current one: 4-bit codes with up to 4 query heads per KV head, where the
// second set of group registers fits the kernel's budget without spills.
template <int G, int QB>
constexpr bool kPrefetchGroups = QB == 4 && G <= 4;

// This wavefront's complete groups g0, g0 + 4 * 64, ... below full_end (a
// multiple of 64; g0 < full_end) as a software pipeline: the next group's loads (and, for
// a paged stream, the page of the group after it) are in flight while a
// group is scored.  The loop body holds no branch around a load.
template <int G, int KB, int QB, bool kPaged>
__device__ __forceinline__ void attend_groups_pipelined(const QSegment& q, int& g0, int full_end, int c,
                                                        const QueryCols<KB, (G + 3) / 4>& qc,
                                                        float qk_scale, uint16_t* p_lds,
                                                        RowState<(G + 3) / 4>& rs, WaveState& st) {
  constexpr int kStep = kWaves * LEANK_QUANT_GROUP;
  const int last = full_end - LEANK_QUANT_GROUP;
  GroupRegs<KB, QB> cur, nxt;
  int page = kPaged ? q.pages[g0 / LEANK_QUANT_GROUP] : 0;
  load_group<KB, QB, true>(q, c, g0, page, cur);
  if (kPaged) page = q.pages[min(g0 + kStep, last) / LEANK_QUANT_GROUP];
  for (; g0 + kStep < full_end; g0 += kStep) {
    load_group<KB, QB, true>(q, c, g0 + kStep, page, nxt);
    if (kPaged) page = q.pages[min(g0 + 2 * kStep, last) / LEANK_QUANT_GROUP];
    attend_group<G, KB, QB>(cur, c, qc, qk_scale, p_lds, rs, st);
    // the copy waits for the next group's loads: keep it after the group's
    // work, where those loads have had the whole group to land
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  }
  attend_group<G, KB, QB>(cur, c, qc, qk_scale, p_lds, rs, st);
  g0 += kStep;  // the wavefront's first group at or past full_end
}

// Whether a wavefront loads only the K part of its next group (K codes and
// parameters, 14 VGPRs at 8 bits) while it scores the current one: 8-bit
// codes with up to 4 query heads per KV head, where the whole next group
// (46 VGPRs) spills at three waves per SIMD.
template <int G, int QB>
constexpr bool kPrefetchGroupK = QB == 8 && G <= 4;

// As attend_groups_pipelined, with only the next group's K codes and
// parameters in flight while a group is scored; its V codes are issued when
// the group is done and land behind the next group's tables and scores.
template <int G, int KB, int QB, bool kPaged>
__device__ __forceinline__ void attend_groups_kpart_pipelined(const QSegment& q, int& g0, int full_end, int c,
                                                    const QueryCols<KB, (G + 3) / 4>& qc,
                                                    float qk_scale, uint16_t* p_lds,
                                                    RowState<(G + 3) / 4>& rs, WaveState& st) {
  constexpr int kStep = kWaves * LEANK_QUANT_GROUP;
  GroupRegs<KB, QB> cur, nxt;
  load_group<KB, QB, true>(q, c, g0, kPaged ? q.pages[g0 / LEANK_QUANT_GROUP] : 0, cur);
  for (; g0 + kStep < full_end; g0 += kStep) {
    const int pn = kPaged ? q.pages[(g0 + kStep) / LEANK_QUANT_GROUP] : 0;
    load_group<KB, QB, true, 1>(q, c, g0 + kStep, pn, nxt);
    attend_group<G, KB, QB>(cur, c, qc, qk_scale, p_lds, rs, st);
    __builtin_amdgcn_sched_barrier(0);
    cur.par = nxt.par;
#pragma unroll
    for (int i = 0; i < KB * QB; ++i) cur.kc[i] = nxt.kc[i];
    cur.vs = nxt.vs;
    cur.vm = nxt.vm;
    load_group<KB, QB, true, 2>(q, c, g0 + kStep, pn, cur);
  }
  attend_group<G, KB, QB>(cur, c, qc, qk_scale, p_lds, rs, st);
  g0 += kStep;
}

// Middle rows [r0, r1) of a low-bit stream (r0 on a group boundary): the
// wavefront's complete groups through the row-per-lane path, then, if it
// takes it, the open group (staged rows) in the 16x16 tile layout, whose
// state the row path's state is first folded into.
template <int G, int KB, int QB>
__device__ __forceinline__ void attend_range_q(const QSegment& q, int r0, int r1, int c,
                                               const u32x4_t (&qa)[KB], const uint16_t* s_q,
                                               const int16_t* s_idx, float qk_scale,
                                               uint16_t* p_lds, WaveState& st, float (&vmin)[4]) {
  constexpr int NQ = (G + 3) / 4;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  int g0 = r0 + wave * LEANK_QUANT_GROUP;
  const int full_end = min(r1, q.full_rows);
  if (g0 < full_end) {
    QueryCols<KB, NQ> qc;
    gather_query_cols<G, KB, NQ>(s_q, s_idx, c, qc);
    RowState<NQ> rs;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rs.m[qd][i] = -INFINITY;
        rs.l[qd][i] = 0.0f;
        rs.vmin[qd][i] = 0.0f;
      }
    }
    if constexpr (kPrefetchGroups<G, QB>) {
      if (q.pool)
        attend_groups_pipelined<G, KB, QB, true>(q, g0, full_end, c, qc, qk_scale, p_lds, rs, st);
      else
        attend_groups_pipelined<G, KB, QB, false>(q, g0, full_end, c, qc, qk_scale, p_lds, rs, st);
    } else if constexpr (kPrefetchGroupK<G, QB>) {
      if (q.pool)
        attend_groups_kpart_pipelined<G, KB, QB, true>(q, g0, full_end, c, qc, qk_scale,
                                                       p_lds, rs, st);
      else
        attend_groups_kpart_pipelined<G, KB, QB, false>(q, g0, full_end, c, qc, qk_scale,
                                                        p_lds, rs, st);
    } else {
      for (; g0 < full_end; g0 += kWaves * LEANK_QUANT_GROUP) {
        GroupRegs<KB, QB> gr;
        load_group<KB, QB, false>(q, c, g0, q.pool ? q.pages[g0 / LEANK_QUANT_GROUP] : 0, gr);
        attend_group<G, KB, QB>(gr, c, qc, qk_scale, p_lds, rs, st);
      }
    }
    // fold into the tile layout: head 4 grp + i of lane (col, grp), whose
    // 16 lanes' sums the record adds up
    const int grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = -INFINITY, l = 0.0f, vm = 0.0f;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        // sums over the four rows of lanes: the 16 lanes of a row then
        // hold the head's total between them
        float lt = rs.l[qd][i], vt = rs.vmin[qd][i];
        lt += __shfl_xor(lt, 16);
        vt += __shfl_xor(vt, 16);
        lt += __shfl_xor(lt, 32);
        vt += __shfl_xor(vt, 32);
        if (grp == qd) {
          m = rs.m[qd][i];
          l = lt;
          vm = vt;
        }
      }
      st.m[i] = m;
      st.l[i] = l;
      vmin[i] = vm;
    }
  }
  for (; g0 < r1; g0 += kWaves * LEANK_QUANT_GROUP) {
    // the open group: staged bf16 rows, the last tile possibly partial
    for (int t0 = g0; t0 < r1 && t0 < g0 + LEANK_QUANT_GROUP; t0 += kTileRows) {
      const int nvalid = r1 - t0;
      QTileRegs<KB, QB> cur;
      load_tile_q<KB, QB>(q, c, t0, nvalid, cur);
      f32x4_t s[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) s[j] = mfma_bf16(qa[kk], cur.kf[j][kk], s[j]);
      }
      if (nvalid >= kTileRows)
        softmax_pv_q<G, QB, false>(s, cur.vc, cur.vs, cur.vm, kTileRows, qk_scale, p_lds, st, vmin);
      else
        softmax_pv_q<G, QB, true>(s, cur.vc, cur.vs, cur.vm, nvalid, qk_scale, p_lds, st, vmin);
    }
  }
}

}  // namespace leank
