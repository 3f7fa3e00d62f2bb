// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "leank.h"

namespace leank {

// ---------------------------------------------------------------- host side

#define LEANK_HIP_TRY(expr)                          \
  do {                                               \
    if ((expr) != hipSuccess) return LEANK_EHIP;     \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// V rows are stored in blocks of LEANK_V_BLOCK rows: a region of `rows` rows
// takes v_rows(rows) rows of storage.
__host__ __device__ inline int64_t v_rows(int64_t rows) {
  return (rows + LEANK_V_BLOCK - 1) / LEANK_V_BLOCK * LEANK_V_BLOCK;
}

// Element offset of (row r, channel ch) inside a V region stored in blocks:
// block r / 8 holds, channel by channel, the 8 rows of that block.
__host__ __device__ inline int64_t v_elem(int64_t r, int ch) {
  return ((r / LEANK_V_BLOCK) * LEANK_HEAD_DIM + ch) * LEANK_V_BLOCK + (r % LEANK_V_BLOCK);
}

// Decomposition of one decode call into work items.  Every (batch row,
// KV head) pair owns n_sl_items items over its full-width rows followed by
// n_mid[h] items over its middle rows; the pairs of one batch row are laid
// out head by head, and batch rows follow each other.  In a fused decode
// step, full-width item 0 of each pair also carries the append (so a step
// has at least one full-width item per pair, even over no cached rows).
struct WorkPlan {
  int32_t group;          // query heads per KV head
  int32_t t_sl;           // valid full-width rows: min(ctx, n_sink + window)
  int32_t t_mid;          // middle rows: max(0, ctx - n_sink - window)
  int32_t n_sl_items;
  int32_t sl_rows;        // rows per full-width item
  int32_t n_mid[LEANK_MAX_KV_HEADS];       // middle items of head h (bulk + tail)
  int32_t mid_rows[LEANK_MAX_KV_HEADS];    // rows per bulk middle item
  int32_t n_mid_b[LEANK_MAX_KV_HEADS];     // bulk middle items (the first ones)
  int32_t mid_rows_t[LEANK_MAX_KV_HEADS];  // rows per tail middle item
  int32_t bulk_per_b;     // items of a batch row dispatched first (full-width + bulk middle)
  int32_t tail_per_b;     // items of a batch row dispatched after every bulk item
  int32_t sl_first;       // 1: every row's full-width items are dispatched before any middle item
  int32_t step;           // 1 for a fused decode step
  int32_t head_base[LEANK_MAX_KV_HEADS + 1];  // first item of head h within a batch row
  int32_t items_per_b;
  int64_t n_items;
  int32_t partial_stride;  // floats per item record
  size_t partial_bytes;
  size_t workspace_bytes;
};

int validate_cache(const leank_layer_cache* c, bool need_buffers);

// In-page layout of a paged low-bit middle: a page holds one 64-row K group
// of every live head -- the K codes of the live heads in group order, then
// their K (scale, min) pairs, then their V code blocks, then their V row
// parameters.  A head at kept-channel prefix P and live rank R starts its K
// codes at byte 64 P bits / 8, its K pairs at kc_bytes + 8 P, its V codes at
// kc_bytes + kp_bytes + R vc_head and its V parameters at kc_bytes +
// kp_bytes + n_live vc_head + R vp_head.
struct QPageLayout {
  int64_t kc_bytes;  // K codes of all live heads
  int64_t kp_bytes;  // their K pairs
  int64_t vc_head;   // V codes of one head: 8 blocks
  int64_t vp_head;   // V parameters of one head: 64 (scale, min) pairs
  int64_t page_bytes;
};
inline QPageLayout q_page_layout(int64_t kept_sum, int64_t n_live, int bits) {
  QPageLayout l;
  l.kc_bytes = LEANK_PAGE_ROWS * kept_sum * bits / 8;
  l.kp_bytes = 8 * kept_sum;
  l.vc_head = static_cast<int64_t>(LEANK_PAGE_ROWS) * LEANK_HEAD_DIM * bits / 8;
  l.vp_head = 8 * LEANK_PAGE_ROWS;
  l.page_bytes = l.kc_bytes + l.kp_bytes + n_live * (l.vc_head + l.vp_head);
  return l;
}
// HBM bytes one middle row of a live head with `kept` channels streams
// (bf16 or low-bit layout, K group parameters not counted).
int64_t middle_row_bytes(const leank_layer_cache* c, int kept);
// ctx_len: cached rows the items cover (0 allowed in a step, step = 1).
int make_work_plan(const leank_layer_cache* c, int64_t ctx_len, int step, WorkPlan* plan);

// ---------------------------------------------------------------- device side

template <int... Is, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, fully unrolled,
// so that i can feed builtins that need an immediate operand.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, static_cast<F&&>(f));
}

// DPP controls of the GCN/CDNA encoding (all act inside a 16-lane row).
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]: lane ^ 1
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]: lane ^ 2
  kDppRowMirror = 0x140,    // lane i <- lane 15 - i
  kDppHalfMirror = 0x141,   // lane i <- lane 7 - i within each half row
  kDppRowNewBcast = 0x150,  // + n: every lane <- lane n of its row
};

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  // every pattern used here reads a valid lane, so no "old" value is needed
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// One lane's word (channels 2 lane, 2 lane + 1) of row r of a V region
// stored in blocks of LEANK_V_BLOCK rows.
__device__ __forceinline__ uint32_t load_v_row_word(const uint16_t* region, int64_t r, int lane) {
  const uint32_t lo = region[v_elem(r, 2 * lane)];
  const uint32_t hi = region[v_elem(r, 2 * lane + 1)];
  return lo | (hi << 16);
}
__device__ __forceinline__ void store_v_row_word(uint16_t* region, int64_t r, int lane, uint32_t w) {
  region[v_elem(r, 2 * lane)] = static_cast<uint16_t>(w & 0xffffu);
  region[v_elem(r, 2 * lane + 1)] = static_cast<uint16_t>(w >> 16);
}

// Word `lane` of a token's compacted K row (kept channels j = 2 lane,
// 2 lane + 1 of the head) from its full row, whose channels 2 m, 2 m + 1
// are held by lane m in `full`.  c0, c1 are the kept channel ids (any
// value in [0, 128) when 2 lane >= kept).  Every lane of the wavefront must
// call it (cross-lane reads).
__device__ __forceinline__ uint32_t compact_k_word(uint32_t full, int c0, int c1) {
  const uint32_t w0 = static_cast<uint32_t>(__shfl(static_cast<int>(full), c0 >> 1));
  const uint32_t w1 = static_cast<uint32_t>(__shfl(static_cast<int>(full), c1 >> 1));
  const uint32_t lo = (c0 & 1) ? (w0 >> 16) : (w0 & 0xffffu);
  const uint32_t hi = (c1 & 1) ? (w1 >> 16) : (w1 & 0xffffu);
  return lo | (hi << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.x*b.x + a.y*b.y + c for two packed bf16 pairs, float32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

}  // namespace leank
