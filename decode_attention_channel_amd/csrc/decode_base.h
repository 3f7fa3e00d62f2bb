// Shared pieces of the decode kernels: the launch parameters, the
// matrix-instruction and cross-lane helpers, and the per-wavefront softmax
// state.  Compile-time knobs (defaults are the measured best on MI355X):
//   LEANK_NT_LOADS   1 = stream K/V with non-temporal loads
#pragma once

#include <math.h>

#include "common.h"
#include "quant.h"

#ifndef LEANK_NT_LOADS
#define LEANK_NT_LOADS 1
#endif

namespace leank {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileRows = 32;
// largest item count per (batch row, KV head) pair that the one-wavefront
// combine merges (larger counts use the workgroup combine)
#ifndef LEANK_WAVE_COMBINE_ITEMS
#define LEANK_WAVE_COMBINE_ITEMS 32
#endif
constexpr int kWaveCombineItems = LEANK_WAVE_COMBINE_ITEMS;
// its reductions cover one or two 16-lane rows of item lanes
static_assert(kWaveCombineItems == 16 || kWaveCombineItems == 32,
              "the one-wavefront combine merges up to 16 or 32 items");
constexpr float kLog2e = 1.4426950408889634f;

// Raw buffer resources (CDNA): word 3 of the descriptor for plain byte
// addressing, the cache-policy operand of a non-temporal load, and an
// offset past any resource's end (its load returns zeros).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kBufNT = LEANK_NT_LOADS ? 2 : 0;
constexpr uint32_t kBufOutside = 0x80000000u;

// The reference max only moves when a tile's max exceeds it by more than
// this (base-2 units), so weights stay <= 2^kRescaleSlack and most tiles
// skip the rescale; the softmax is unchanged because the reference cancels.
constexpr float kRescaleSlack = 8.0f;

struct DecodeHead {
  int64_t k_off;   // elements of K_prun, -1 for a dead head (low-bit: kept channels of the live heads before it)
  int64_t v_off;   // elements of V_mid, -1 for a dead head (low-bit: its rank among the live heads)
  int32_t kept;
  int32_t n_mid;     // middle items of this head per batch row (bulk + tail)
  int32_t mid_rows;  // rows per bulk middle item
  int32_t base;      // first item of this head within a batch row
  int32_t n_mid_b;     // bulk middle items (chunks [0, n_mid_b)); the rest are tail items
  int32_t mid_rows_t;  // rows per tail middle item
  // paged low-bit middle: byte offsets of the head's K codes, K pairs, V
  // codes and V parameters within a page
  int32_t pq_k_codes, pq_k_par, pq_v_codes, pq_v_par;
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
  int32_t lens_from_pos;  // 1: row b attends over row_pos[b] + 1 tokens (appended before the call's kernels)
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
  int32_t wave_items;  // one-wavefront combine: the most items of any pair
  // dispatch order: every batch row's bulk items (its full-width and bulk
  // middle items, head by head), then every batch row's tail items
  int32_t bulk_per_b;
  int32_t tail_per_b;
  int64_t n_bulk;  // batch * bulk_per_b
  int64_t n_sl_all;  // full-width items dispatched first (batch * n_kv * n_sl_items), or 0
  // calls of at most 8 KV heads: each head's last item + 1 within a batch
  // row's bulk items (full-width and bulk middle together, or bulk middle
  // only when n_sl_all > 0) and within its tail items, cumulative over the
  // heads (entries past n_kv - 1 hold INT32_MAX), so an item finds its head
  // from values loaded with the other parameters
  int32_t bulk_end8[8];
  int32_t tail_end8[8];
  DecodeHead heads[LEANK_MAX_KV_HEADS];
};
// kernel arguments are limited to 4 KiB
static_assert(sizeof(DecodeParams) <= 4096, "decode launch parameters exceed the kernel argument limit");

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// LDS staging is written in 16- or 32-bit pieces and read back as vectors:
// these types may alias any other, so no access is reordered across them
typedef uint32_t u32x4_alias_t __attribute__((ext_vector_type(4), may_alias));
typedef uint32_t u32x2_alias_t __attribute__((ext_vector_type(2), may_alias));
typedef float f32x4_alias_t __attribute__((ext_vector_type(4), may_alias));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// This lane's wavefront within the workgroup, in a scalar register.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

#ifndef LEANK_TOUCH_ARGS
#define LEANK_TOUCH_ARGS 1
#endif
// Reads one dword of every 64-byte line of the first `kLines` lines of the
// kernel argument block and waits for them, so that the lines sit in the
// scalar cache before the kernel's own argument loads.  Those loads form a
// chain (the item's head depends on the per-head counts, its record on the
// head, its stream addresses on both), and each first touch of a line
// missed the cache at every step: per-item timestamps (a one-round
// 128K-token layer) put the item's head record 1.1 us after its start and
// its staging loads 2.5 us after it, 0.4 and 1.3 us with the lines touched
// first (Llama batch-64 4K step 110.9 -> 110.1 us, Qwen2.5-7B-shaped
// batch-16 32K 89.5 -> 88.8 us, 32-layer 128K-token batch-1 token 958 ->
// 940 us).  Loads only; the values are discarded.
template <int kLines, class Args>
__device__ __forceinline__ void touch_kernarg_lines() {
  static_assert(kLines >= 1 && kLines <= 16, "touch at most 16 lines");
  static_assert(sizeof(Args) >= kLines * 64, "the touched lines must lie inside the argument block");
  const auto* args = __builtin_amdgcn_kernarg_segment_ptr();
  uint32_t sink;
  asm volatile(
      "s_load_dword %0, %1, 0x0\n\t"
      ".if %2 > 1\n\ts_load_dword %0, %1, 0x40\n\t.endif\n\t"
      ".if %2 > 2\n\ts_load_dword %0, %1, 0x80\n\t.endif\n\t"
      ".if %2 > 3\n\ts_load_dword %0, %1, 0xc0\n\t.endif\n\t"
      ".if %2 > 4\n\ts_load_dword %0, %1, 0x100\n\t.endif\n\t"
      ".if %2 > 5\n\ts_load_dword %0, %1, 0x140\n\t.endif\n\t"
      ".if %2 > 6\n\ts_load_dword %0, %1, 0x180\n\t.endif\n\t"
      ".if %2 > 7\n\ts_load_dword %0, %1, 0x1c0\n\t.endif\n\t"
      ".if %2 > 8\n\ts_load_dword %0, %1, 0x200\n\t.endif\n\t"
      ".if %2 > 9\n\ts_load_dword %0, %1, 0x240\n\t.endif\n\t"
      ".if %2 > 10\n\ts_load_dword %0, %1, 0x280\n\t.endif\n\t"
      ".if %2 > 11\n\ts_load_dword %0, %1, 0x2c0\n\t.endif\n\t"
      ".if %2 > 12\n\ts_load_dword %0, %1, 0x300\n\t.endif\n\t"
      ".if %2 > 13\n\ts_load_dword %0, %1, 0x340\n\t.endif\n\t"
      ".if %2 > 14\n\ts_load_dword %0, %1, 0x380\n\t.endif\n\t"
      ".if %2 > 15\n\ts_load_dword %0, %1, 0x3c0\n\t.endif\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(sink)
      : "s"(args), "i"(kLines)
      : "memory");
}

// A 64-bit value that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

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

// A operand of the score product for this lane: query head col of the
// group, kept channels 32 kk + 8 grp .. +7 (zero past c or for col >= G).
template <int G, int KB>
__device__ __forceinline__ void gather_q(const uint16_t* s_q, const int16_t* s_idx, bool dense,
                                         int c, u32x4_t (&qa)[KB]) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  if (dense && c == LEANK_HEAD_DIM) {
    // all channels: one 16-byte LDS read per block
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
      qa[kk] = col < G ? *reinterpret_cast<const u32x4_alias_t*>(s_q + col * LEANK_HEAD_DIM + 32 * kk + 8 * grp)
                       : u32x4_t{0u, 0u, 0u, 0u};
    return;
  }
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

}  // namespace leank
