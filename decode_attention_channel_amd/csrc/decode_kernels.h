// Device code of leank_decode_attn: single-token decode attention over the
// channel-pruned cache (LeanK page, section 3.1 item 3 and section 3.2; GQA
// as in section 5.2.3 of the KV-pruning white paper; scale as in FastGen
// page 5.3).
//
// Work items.  Each (batch row b, KV head h) pair is split into items over
// its full-width rows (K_sl/V_sl, 128 channels) and, for a live head, over
// its middle rows (K_prun with the head's kept channels c, V_mid).  One
// 256-thread workgroup runs one item; its 4 wavefronts take 32-row tiles
// round-robin (whole 64-row K groups in a low-bit middle).  All G query
// heads of the group share every K and V load.
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
// Pieces: decode_base.h (parameters, helpers), tile_bf16.h (bf16 tiles),
// tile_lowbit.h (low-bit middle tiles), step_tokens.h (the fused step's
// append).  Compile-time knob here: LEANK_WAVES_PER_EU, the register budget
// hint for the split kernel (0 = none).

#pragma once

#include "decode_base.h"
#include "step_tokens.h"
#include "tile_bf16.h"
#include "tile_lowbit.h"

#ifndef LEANK_WAVES_PER_EU
#define LEANK_WAVES_PER_EU 3
#endif
#ifndef LEANK_Q_WAVES_PER_EU
#define LEANK_Q_WAVES_PER_EU 2
#endif
// register budget: LEANK_WAVES_PER_EU for bf16 caches and for low-bit
// middle streams whose live heads keep at most 32 channels;
// LEANK_Q_WAVES_PER_EU for wider low-bit heads (their scaled query
// operands and code tiles keep more registers live)
#if LEANK_WAVES_PER_EU
#define LEANK_SPLIT_ATTRS                  \
  __launch_bounds__(kThreads) __attribute__( \
      (amdgpu_waves_per_eu(QB && KBMAX > 1 ? LEANK_Q_WAVES_PER_EU : LEANK_WAVES_PER_EU)))
#else
#define LEANK_SPLIT_ATTRS __launch_bounds__(kThreads)
#endif

namespace leank {

// Rows [r0, r1) of middle chunk `chunk` of a head (t_mid middle rows in the
// batch row): bulk chunks [0, n_mid_b) of mid_rows rows, then tail chunks of
// mid_rows_t rows.
__device__ __forceinline__ void mid_chunk_rows(const DecodeHead& hd, int chunk, int t_mid, int& r0,
                                               int& r1) {
  if (chunk < hd.n_mid_b) {
    r0 = chunk * hd.mid_rows;
    r1 = r0 + hd.mid_rows;
  } else {
    r0 = hd.n_mid_b * hd.mid_rows + (chunk - hd.n_mid_b) * hd.mid_rows_t;
    r1 = r0 + hd.mid_rows_t;
  }
  r1 = min(t_mid, r1);
}

// Middle rows of item `chunk_id` of head hd in batch row b (t_mid middle
// rows in this row) of a low-bit stream: the head's kept channels select
// the tile width (bf16 middles: attend_middle_staged).
template <int G, int QB, int KBMAX>
__device__ __forceinline__ void attend_middle(const DecodeParams& p, const DecodeHead& hd, int b,
                                              int chunk_id, int t_mid, const uint16_t* s_q,
                                              const int16_t* s_idx, const int32_t* s_pages,
                                              uint16_t* p_lds, WaveState& st, float (&vmin)[4]) {
  int r0, r1;
  mid_chunk_rows(hd, chunk_id, t_mid, r0, r1);
  const int c = hd.kept;
  if constexpr (QB != 0) {
    const QSegment q = q_segment<QB>(p, hd, b, t_mid);
    const int kb = (c + 31) / 32;
    if (KBMAX == 1 || kb == 1) {
      u32x4_t qa[1];
      gather_q<G, 1>(s_q, s_idx, false, c, qa);
      attend_range_q<G, 1, QB>(q, r0, r1, c, qa, s_q, s_idx, p.qk_scale, p_lds, st, vmin);
    } else if constexpr (KBMAX >= 2) {
      if (KBMAX == 2 || kb == 2) {
        u32x4_t qa[2];
        gather_q<G, 2>(s_q, s_idx, false, c, qa);
        attend_range_q<G, 2, QB>(q, r0, r1, c, qa, s_q, s_idx, p.qk_scale, p_lds, st, vmin);
      } else if constexpr (KBMAX >= 3) {
        if (kb == 3) {
          u32x4_t qa[3];
          gather_q<G, 3>(s_q, s_idx, false, c, qa);
          attend_range_q<G, 3, QB>(q, r0, r1, c, qa, s_q, s_idx, p.qk_scale, p_lds, st, vmin);
        } else {
          u32x4_t qa[4];
          gather_q<G, 4>(s_q, s_idx, false, c, qa);
          attend_range_q<G, 4, QB>(q, r0, r1, c, qa, s_q, s_idx, p.qk_scale, p_lds, st, vmin);
        }
      }
    }
  }
}

// bf16 middle rows of item `chunk_id` of a paged stream (holds the
// workgroup barrier that publishes q, the kept ids and the item's pages,
// which the caller has staged).
template <int G>
__device__ __forceinline__ void attend_middle_paged(const DecodeParams& p, const DecodeHead& hd,
                                                    int b, int chunk_id, int t_mid,
                                                    const uint16_t* s_q, const int16_t* s_idx,
                                                    const int32_t* s_pages, uint16_t* p_lds,
                                                    WaveState& st) {
  int r0, r1;
  mid_chunk_rows(hd, chunk_id, t_mid, r0, r1);
  const int c = hd.kept;
  const int32_t* g_pages =
      p.block_table + static_cast<int64_t>(b) * p.pages_per_row + r0 / LEANK_PAGE_ROWS;
  switch ((c + 31) / 32) {
    case 1:
      attend_range_paged_staged<G, 1>(p.pool, p.page_elems, g_pages, s_pages, hd.k_off, hd.v_off,
                                      r0, r1, c, s_q, s_idx, p.qk_scale, p_lds, st);
      break;
    case 2:
      attend_range_paged_staged<G, 2>(p.pool, p.page_elems, g_pages, s_pages, hd.k_off, hd.v_off,
                                      r0, r1, c, s_q, s_idx, p.qk_scale, p_lds, st);
      break;
    case 3:
      attend_range_paged_staged<G, 3>(p.pool, p.page_elems, g_pages, s_pages, hd.k_off, hd.v_off,
                                      r0, r1, c, s_q, s_idx, p.qk_scale, p_lds, st);
      break;
    default:
      attend_range_paged_staged<G, 4>(p.pool, p.page_elems, g_pages, s_pages, hd.k_off, hd.v_off,
                                      r0, r1, c, s_q, s_idx, p.qk_scale, p_lds, st);
      break;
  }
}

// bf16 middle rows of item `chunk_id` of a contiguous stream; `stage` is
// the workgroup's staging (see attend_range_staged).
template <int G, class Stage>
__device__ __forceinline__ void attend_middle_contig(const DecodeParams& p, const DecodeHead& hd,
                                                     int b, int chunk_id, int t_mid,
                                                     const uint16_t* s_q, const int16_t* s_idx,
                                                     uint16_t* p_lds, WaveState& st, Stage&& stage) {
  int r0, r1;
  mid_chunk_rows(hd, chunk_id, t_mid, r0, r1);
  const int c = hd.kept;
  const uint16_t* kb = p.k_prun + hd.k_off + static_cast<int64_t>(b) * p.mid_cap * c;
  const uint16_t* vb = p.v_mid + hd.v_off + static_cast<int64_t>(b) * p.v_mid_rows * LEANK_HEAD_DIM;
  switch ((c + 31) / 32) {
    case 1:
      attend_range_staged<G, 1>(kb, c, vb, r0, r1, -1, c, s_q, s_idx, false, p.qk_scale, p_lds, st, stage);
      break;
    case 2:
      attend_range_staged<G, 2>(kb, c, vb, r0, r1, -1, c, s_q, s_idx, false, p.qk_scale, p_lds, st, stage);
      break;
    case 3:
      attend_range_staged<G, 3>(kb, c, vb, r0, r1, -1, c, s_q, s_idx, false, p.qk_scale, p_lds, st, stage);
      break;
    default:
      attend_range_staged<G, 4>(kb, c, vb, r0, r1, -1, c, s_q, s_idx, false, p.qk_scale, p_lds, st, stage);
      break;
  }
}

// The head of item r of a batch row's phase, from the heads' cumulative
// ends (nondecreasing, INT32_MAX past the last head): h = the number of
// ends at or below r, r becomes the item's place within its head.  All
// compares and selects, no dependent load: the ends come with the launch
// parameters.
__device__ __forceinline__ void head_from_ends(const int32_t (&end)[8], int& r, int& h) {
  int start = 0, hh = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const bool past = r >= end[i];
    hh += past ? 1 : 0;
    start = past ? end[i] : start;
  }
  h = hh;
  r -= start;
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
  // per wavefront: the weight staging of a tile (low-bit: of a 64-row group,
  // and that group's parameter and query tables)
  __shared__ __attribute__((aligned(16))) uint16_t s_p[kWaves][QB ? group_lds_halves<KBMAX, G>() : 2 * 16 * kTileRows];
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

  // bring the launch parameters' scalar fields and the first 8 heads'
  // records (their first 14 lines) into the scalar cache
  static_assert(offsetof(DecodeParams, heads) + 8 * sizeof(DecodeHead) <= 14 * 64,
                "touched lines do not cover the first 8 heads");
  if (LEANK_TOUCH_ARGS) touch_kernarg_lines<14, DecodeParams>();

  // dispatch order: every batch row's bulk items (full-width, then bulk
  // middle, head by head; or, when the plan puts the full-width items
  // first, every row's full-width items, then every row's bulk middle
  // items), then every batch row's tail items; `local` is the item's place
  // among its pair's records (full-width items, then middle chunks in row
  // order), so the record order does not depend on it
  // (32-bit arithmetic: a launch holds fewer than 2^31 items; the results
  // go through readfirstlane so that they stay in scalar registers)
  const uint32_t item = blockIdx.x;
  int b, h = 0, local;
  if (item < static_cast<uint32_t>(p.n_sl_all)) {
    const uint32_t per_b = static_cast<uint32_t>(p.n_kv * p.n_sl_items);
    b = static_cast<int>(item / per_b);
    const int r = static_cast<int>(item - static_cast<uint32_t>(b) * per_b);
    h = r / p.n_sl_items;
    local = r - h * p.n_sl_items;
  } else if (item < static_cast<uint32_t>(p.n_bulk)) {
    // every row's bulk middle items after the full-width ones (n_sl_all > 0),
    // or each row's full-width and bulk middle items together
    const uint32_t n_sl = p.n_sl_all > 0 ? 0u : static_cast<uint32_t>(p.n_sl_items);
    const uint32_t per_b = static_cast<uint32_t>(p.bulk_per_b) -
                           (p.n_sl_all > 0 ? static_cast<uint32_t>(p.n_kv * p.n_sl_items) : 0u);
    const uint32_t j = item - static_cast<uint32_t>(p.n_sl_all);
    b = static_cast<int>(j / per_b);
    int r = static_cast<int>(j - static_cast<uint32_t>(b) * per_b);
    if (p.n_kv <= 8) {
      head_from_ends(p.bulk_end8, r, h);
    } else {
      while (h + 1 < p.n_kv && r >= static_cast<int>(n_sl) + p.heads[h].n_mid_b) {
        r -= static_cast<int>(n_sl) + p.heads[h].n_mid_b;
        ++h;
      }
    }
    local = r + (p.n_sl_all > 0 ? p.n_sl_items : 0);
  } else {
    const uint32_t t_item = item - static_cast<uint32_t>(p.n_bulk);
    b = static_cast<int>(t_item / static_cast<uint32_t>(p.tail_per_b));
    int r = static_cast<int>(t_item - static_cast<uint32_t>(b) * static_cast<uint32_t>(p.tail_per_b));
    if (p.n_kv <= 8) {
      head_from_ends(p.tail_end8, r, h);
    } else {
      while (h + 1 < p.n_kv && r >= p.heads[h].n_mid - p.heads[h].n_mid_b) {
        r -= p.heads[h].n_mid - p.heads[h].n_mid_b;
        ++h;
      }
    }
    local = p.n_sl_items + p.heads[h].n_mid_b + r;
  }
  b = __builtin_amdgcn_readfirstlane(b);
  h = __builtin_amdgcn_readfirstlane(h);
  local = __builtin_amdgcn_readfirstlane(local);
  const DecodeHead hd = p.heads[h];
  const int64_t rec_item = static_cast<int64_t>(b) * p.items_per_b + hd.base + local;
  const bool middle = local >= p.n_sl_items;
  const bool carries_step = p.step && local == 0;  // block-uniform
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = wave_id();

  const int64_t pair = static_cast<int64_t>(b) * p.n_kv + h;
  // (values read per batch row go through readfirstlane: they are the same
  // in every lane, and scalar registers keep them out of the vector budget)
  int t_sl = p.t_sl, t_mid = p.t_mid;
  int excl = -1;  // ring row replaced by a fused step's append
  if (p.step) {
    // rows cached before the append; the row of the token leaving the
    // window is scored by the step item
    const int64_t pos = p.row_pos ? uniform64(p.row_pos[b]) : p.step_pos;
    const bool ok = pos >= 0 && pos <= p.max_len;
    const int len = ok ? static_cast<int>(pos) : 0;
    if (ok && p.window > 0 && len - p.window >= p.n_sink)
      excl = p.n_sink + (len - p.n_sink) % p.window;
    t_sl = min(len, p.slots);
    t_mid = max(0, len - p.slots);
  } else if (p.ctx_lens) {  // ragged batch: this row may hold fewer tokens than the plan
    const int len = min(max(__builtin_amdgcn_readfirstlane(p.ctx_lens[b]), 0), p.max_len);
    t_sl = min(len, p.slots);
    t_mid = max(0, len - p.slots);
  } else if (p.lens_from_pos) {  // ragged step whose appends ran first
    const int64_t pos = uniform64(p.row_pos[b]);
    const int len = pos >= 0 && pos < p.max_len ? static_cast<int>(pos) + 1 : 0;
    t_sl = min(len, p.slots);
    t_mid = max(0, len - p.slots);
  }
  StepTokens tok{};
  // The workgroup's staging: the group's q rows and the head's kept ids,
  // the item's pages (paged middle) and cleared P staging, in two parts:
  // `stage` issues the global loads into registers and returns the part
  // that writes them to LDS.  The bf16 attend paths issue their first
  // tile's loads between the two, so that a wavefront's staging loads and
  // tile loads are in flight together (written out in one part, a
  // wavefront's tile loads waited for its staging loads' round trip); the
  // workgroup barrier that publishes the staging sits in the attend call
  // (bf16 streams) or just below (low-bit middles).  Where it is written
  // changes the register allocation of the whole kernel: this form
  // measured fastest (written out once before the paths, the Llama
  // batch-64 4K step took 115.4 us instead of 110.9).
  auto stage = [&]() {
    const u32x4_t zero4{0u, 0u, 0u, 0u};
    const bool has_q = t < G * 16;
    const bool has_idx = (middle || carries_step) && t >= 128 && t < 144;
    bool has_page = false;
    u32x4_t qv = zero4, iv = zero4;
    int32_t page = 0;
    if (has_q) {
      const uint16_t* qh = p.q + (static_cast<int64_t>(b) * p.n_q + h * G) * LEANK_HEAD_DIM;
      qv = *reinterpret_cast<const u32x4_t*>(qh + t * 8);
    }
    if (QB == 0 && p.paged && middle && t >= 192) {
      // the item's pages (items span at most 64 pages: their rows are capped
      // by the plan's largest item size)
      int pr0, pr1;
      mid_chunk_rows(hd, local - p.n_sl_items, INT32_MAX, pr0, pr1);
      const int first = pr0 / LEANK_PAGE_ROWS;
      const int i = t - 192;
      has_page = i < (pr1 - pr0) / LEANK_PAGE_ROWS && first + i < p.pages_per_row;
      if (has_page) page = p.block_table[static_cast<int64_t>(b) * p.pages_per_row + first + i];
    }
    if (has_idx)
      iv = *reinterpret_cast<const u32x4_t*>(p.kept_idx + h * LEANK_HEAD_DIM + (t - 128) * 8);
    return [=]() {
      if (has_q) *reinterpret_cast<u32x4_t*>(s_q + t * 8) = qv;
      if (has_page) s_pages[t - 192] = page;
      if (has_idx) *reinterpret_cast<u32x4_t*>(s_idx + (t - 128) * 8) = iv;
      for (int k = lane; k < (QB ? group_lds_halves<KBMAX, G>() : 2 * 16 * kTileRows) / 8; k += 64)
        reinterpret_cast<u32x4_t*>(s_p[wave])[k] = zero4;
    };
  };
  // the item that carries a fused step stages its tokens and V blocks
  // before anything else (one item per pair)
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
          const QGroup at = q_group<QB>(qs, hd.kept, tok.mid_row / LEANK_QUANT_GROUP);
          constexpr int kBlkBytes = LEANK_HEAD_DIM * LEANK_V_BLOCK * QB / 8;
          if (c * 16 < kBlkBytes)
            x = *reinterpret_cast<const u32x4_t*>(
                at.v_codes + ((tok.mid_row % LEANK_QUANT_GROUP) / LEANK_V_BLOCK) * kBlkBytes + c * 16);
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

  if (!middle) {
    const int r0 = local * p.sl_rows;
    const int r1 = min(t_sl, r0 + p.sl_rows);
    const uint16_t* kb = p.k_sl + pair * p.slots * LEANK_HEAD_DIM;
    const uint16_t* vb = p.v_sl + pair * p.v_sl_rows * LEANK_HEAD_DIM;
    attend_range_staged<G, 4>(kb, LEANK_HEAD_DIM, vb, r0, r1, excl, LEANK_HEAD_DIM, s_q, s_idx,
                              true, p.qk_scale, p_lds, st, stage);
  } else if (QB == 0 && !p.paged) {
    attend_middle_contig<G>(p, hd, b, local - p.n_sl_items, t_mid, s_q, s_idx, p_lds, st, stage);
  } else if (QB == 0) {
    stage()();
    attend_middle_paged<G>(p, hd, b, local - p.n_sl_items, t_mid, s_q, s_idx, s_pages, p_lds, st);
  } else {
    stage()();
    __syncthreads();
    attend_middle<G, QB, KBMAX>(p, hd, b, local - p.n_sl_items, t_mid, s_q, s_idx, s_pages, p_lds,
                                st, vmin);
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
  float* rec = p.partials + rec_item * p.partial_stride;
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

  // The append below rewrites the staged blocks in LDS (wavefront 0 sets
  // the appended row of each channel), and every wavefront's part of the
  // record above reads the leaving token's V from the same staged ring
  // block: all of them finish before wavefront 0 starts.
  if (carries_step) __syncthreads();  // block-uniform
  if (carries_step && tok.ok && wave == 0) {
    // the append; this workgroup's reads of the ring row ended before the
    // merge, and no other item of the call uses the rows written here.
    // Lane `lane` owns channels 2 lane, 2 lane + 1: their K words and the
    // 16-byte groups of the two V blocks, so no lane reads another's LDS.
    //
    // Invariant of the whole-block V stores below: each 8-row V block (and,
    // 4-bit, each code byte shared by two rows) is written back with every
    // row but the appended one unchanged -- exactly the bytes this item read
    // in its prologue.  Other items of the call may read the same block at
    // the same time (the last middle item reads the rows before the new
    // middle row; a regular full-width item the ring rows around the
    // slot); they read only rows whose bytes this store leaves as they
    // were, and they mask the one row that changes.  So a block must
    // belong to one (batch row, head) pair and one call must not append to
    // it twice: distinct block-table pages and one step per call keep it so.
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
        const QGroup at = q_group<QB>(qs, hd.kept, r / LEANK_QUANT_GROUP);
        const int r_in = r % LEANK_QUANT_GROUP;
        if (lane < kBlkBytes / 16)
          reinterpret_cast<u32x4_t*>(const_cast<uint8_t*>(at.v_codes) + (r_in / LEANK_V_BLOCK) * kBlkBytes)[lane] =
              reinterpret_cast<const u32x4_t*>(s_vblk[1])[lane];
        if (lane == 0)
          *reinterpret_cast<float2*>(const_cast<float*>(at.v_par) + r_in * 2) = make_float2(s_vpar[0], s_vpar[1]);
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
// with one wavefront, for pairs of at most kWaveCombineItems items: every
// load is issued up front (each lane's two channels of every item, and lane
// i's maximum and weight sum of item i), so the merge takes one round trip
// to memory; the 16-lane row reductions (two rows for 32 items) and the
// weighted sum over the items in item order follow, with no LDS or barrier.  Grid: one workgroup of G
// wavefronts per pair (wavefront g: query head g), so the pair's head
// fields come through scalar loads.  NI (4, 8, 16 or 32) covers the most
// items of any pair of the call: loads past a pair's items re-read its last
// one, so a smaller NI issues fewer of them (Llama batch-64 step: 113.7 ->
// 113.05 us with NI 4 instead of 16).  Up to 32 items this form beats the
// workgroup combine (Qwen batch-16 32K step, 27 items per pair: 93.2 ->
// 92.6 us).
template <int G, int NI>
__global__ __launch_bounds__(64 * G) void decode_combine_wave_kernel(const DecodeParams p) {
  // as in the split kernel (the 32-layer 128K-token token: 938.7 -> 935.0 us)
  if (LEANK_TOUCH_ARGS) touch_kernarg_lines<14, DecodeParams>();
  const int lane = threadIdx.x & 63;
  const int g = threadIdx.x >> 6;
  const int b = static_cast<int>(blockIdx.x / p.n_kv);
  const int h = static_cast<int>(blockIdx.x - b * p.n_kv);
  const DecodeHead hd = p.heads[h];
  const int n_items = p.n_sl_items + hd.n_mid;  // at most NI
  const int64_t stride = p.partial_stride;
  const float* first = p.partials + (static_cast<int64_t>(b) * p.items_per_b + hd.base) * stride;
  const int m_off = G * LEANK_HEAD_DIM + g;
  const int l_off = G * LEANK_HEAD_DIM + G + g;

  float* out = p.out + (static_cast<int64_t>(b) * p.n_q + h * G + g) * LEANK_HEAD_DIM + 2 * lane;
  if (n_items == 0) {  // no rows: zeros
    *reinterpret_cast<float2*>(out) = make_float2(0.0f, 0.0f);
    return;
  }
  // Loads past the pair's items re-read its last item (their weights are
  // 0), so that none of them takes a branch.
  const int last = n_items - 1;
  const float* acc = first + g * LEANK_HEAD_DIM + 2 * lane;
  float2 v[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u)
    v[u] = *reinterpret_cast<const float2*>(acc + min(u, last) * stride);
  const bool has = lane < n_items;
  const float m_ld = first[min(lane, last) * stride + m_off];
  const float l_ld = first[min(lane, last) * stride + l_off];
  const float m_i = has ? m_ld : -INFINITY;
  const float l_i = has ? l_ld : 0.0f;

  // items sit in lanes 0..NI-1: one 16-lane row, or two for NI = 32
  const float m_r = row_max16(m_i);
  const float m_all =
      NI <= 16 ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(m_r)))
               : fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_r), 0)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_r), 16)));
  const float m_use = m_all == -INFINITY ? 0.0f : m_all;
  const float w_i = has ? fast_exp2(m_i - m_use) : 0.0f;
  const float t_r = row_sum16(w_i * l_i);
  const float total =
      NI <= 16 ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t_r)))
               : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t_r), 0)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t_r), 16));
  float2 a = make_float2(0.0f, 0.0f);
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_i), u));  // 0 past the items
    a.x = fmaf(v[u].x, w, a.x);
    a.y = fmaf(v[u].y, w, a.y);
  }
  const float inv = total > 0.0f ? 1.0f / total : 0.0f;  // an empty row gives zeros
  *reinterpret_cast<float2*>(out) = make_float2(a.x * inv, a.y * inv);
}

// Merges the records of one (batch row, KV head) pair for one query head g
// of its group -- or, when the pair has many items, for one of `slices`
// channel slices of that head -- and writes the output.  Threads form
// item groups x float4 channel quads; item group j merges items j,
// j + groups, ... in one pass with a running maximum, and the groups'
// (max, sum, acc) are then merged in a fixed order (across lanes, then
// across wavefronts), so the result does not depend on timing.  Grid:
// pairs x G x slices.
// records a combine thread loads per round trip: a slice holds up to 64
// records per pair, 8 per thread, so one round covers them (measured on the
// 128K-token batch-1 layer: 20.4 us per step against 20.75 us with 4)
#ifndef LEANK_COMBINE_UNROLL
#define LEANK_COMBINE_UNROLL 8
#endif
constexpr int kCombineUnroll = LEANK_COMBINE_UNROLL;

template <int G>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(const DecodeParams p) {
  if (LEANK_TOUCH_ARGS) touch_kernarg_lines<14, DecodeParams>();  // as in the split kernel
  __shared__ float s_max[kWaves * 32];
  __shared__ float4 s_acc[kWaves * 32];
  __shared__ float s_sum[kWaves * 32];
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
  const int grp = t / quads;
  const int quad = t - grp * quads;
  const int ch = g * LEANK_HEAD_DIM + (slice * quads + quad) * 4;

  // one pass: this thread's items n = grp, grp + groups, ... (all their
  // loads issued together) merged with a running maximum
  float m = -INFINITY, l = 0.0f;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int n0 = grp; n0 < n_items; n0 += kCombineUnroll * groups) {
    float mi[kCombineUnroll], li[kCombineUnroll];
    float4 v[kCombineUnroll];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const int n = n0 + u * groups;
      const float* rn = first + static_cast<int64_t>(n < n_items ? n : n0) * stride;
      mi[u] = n < n_items ? rn[m_off] : -INFINITY;
      li[u] = rn[l_off];
      v[u] = *reinterpret_cast<const float4*>(rn + ch);
    }
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const float mn = fmaxf(m, mi[u]);
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float fo = fast_exp2(m - mu), fi = fast_exp2(mi[u] - mu);  // 0 for -inf
      a.x = fmaf(v[u].x, fi, a.x * fo);
      a.y = fmaf(v[u].y, fi, a.y * fo);
      a.z = fmaf(v[u].z, fi, a.z * fo);
      a.w = fmaf(v[u].w, fi, a.w * fo);
      l = fmaf(li[u], fi, l * fo);
      m = mn;
    }
  }
  // the item groups' parts, merged as a fixed tree: first across the
  // lanes of each wavefront (groups quads lanes apart), then the four
  // wavefronts' parts in order through LDS
  for (int off = quads; off < 64; off *= 2) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    float4 x;
    x.x = __shfl_xor(a.x, off);
    x.y = __shfl_xor(a.y, off);
    x.z = __shfl_xor(a.z, off);
    x.w = __shfl_xor(a.w, off);
    const float mn = fmaxf(m, m2);
    const float mu = mn == -INFINITY ? 0.0f : mn;
    const float f1 = fast_exp2(m - mu), f2 = fast_exp2(m2 - mu);
    a.x = fmaf(x.x, f2, a.x * f1);
    a.y = fmaf(x.y, f2, a.y * f1);
    a.z = fmaf(x.z, f2, a.z * f1);
    a.w = fmaf(x.w, f2, a.w * f1);
    l = fmaf(l2, f2, l * f1);
    m = mn;
  }
  const int wave = t >> 6;
  const int lane = t & 63;
  if (lane < quads) {
    s_max[wave * quads + lane] = m;
    s_acc[wave * quads + lane] = a;
    s_sum[wave * quads + lane] = l;
  }
  __syncthreads();
  if (t < quads) {
    float mw[kWaves];
    float mn = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = s_max[w * quads + t];
      mn = fmaxf(mn, mw[w]);
    }
    const float mu = mn == -INFINITY ? 0.0f : mn;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float total = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(mw[w] - mu);
      const float4 x = s_acc[w * quads + t];
      o.x = fmaf(x.x, f, o.x);
      o.y = fmaf(x.y, f, o.y);
      o.z = fmaf(x.z, f, o.z);
      o.w = fmaf(x.w, f, o.w);
      total = fmaf(s_sum[w * quads + t], f, total);
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
  if (p.combine_slices == 0) {  // every pair has at most kWaveCombineItems items
    const dim3 pairs(static_cast<unsigned>(n_pairs));
    if (p.wave_items <= 4)
      hipLaunchKernelGGL((decode_combine_wave_kernel<G, 4>), pairs, dim3(64 * G), 0, s, p);
    else if (p.wave_items <= 8)
      hipLaunchKernelGGL((decode_combine_wave_kernel<G, 8>), pairs, dim3(64 * G), 0, s, p);
    else if (p.wave_items <= 16)
      hipLaunchKernelGGL((decode_combine_wave_kernel<G, 16>), pairs, dim3(64 * G), 0, s, p);
    else
      hipLaunchKernelGGL((decode_combine_wave_kernel<G, kWaveCombineItems>), pairs, dim3(64 * G), 0, s, p);
  } else {
    hipLaunchKernelGGL(decode_combine_kernel<G>,
                       dim3(static_cast<unsigned>(n_pairs * G * p.combine_slices)), dim3(kThreads),
                       0, s, p);
  }
  LEANK_HIP_TRY(hipGetLastError());
  return LEANK_OK;
}

}  // namespace leank
