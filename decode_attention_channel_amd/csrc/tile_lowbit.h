// Tiles of the low-bit middle streams (K codes per channel over 64-row
// groups, V codes per token).
#pragma once

#include "decode_base.h"

namespace leank {

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

}  // namespace leank
