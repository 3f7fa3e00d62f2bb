// Low-bit middle streams: parameters of the packing kernels and the host
// hooks leank_pack_k calls for a cache planned by leank_plan_layer_q.
#pragma once

#include "common.h"

namespace leank {

struct QuantHead {
  int64_t k_q_off;      // bytes
  int64_t k_qp_off;     // floats
  int64_t k_stage_off;  // elements
  int64_t v_q_off;      // bytes
  int64_t v_qp_off;     // floats
  int32_t kept;
  int32_t pad;
};

struct QuantParams {
  const uint16_t* k_src;  // bf16 [B][H_kv][n_src][128]
  const uint16_t* v_src;
  int64_t n_src;
  uint8_t* k_q;
  float* k_qp;
  uint16_t* k_stage;
  uint8_t* v_q;
  float* v_qp;
  uint16_t* k_sl;
  uint16_t* v_sl;
  const int16_t* kept_idx;
  int64_t mid_cap;
  int64_t g_rows;      // K code rows per (b, head): whole groups
  int64_t v_rows_cap;  // V code rows per (b, head): whole blocks
  int64_t v_sl_rows;
  int64_t t_mid;       // bulk: middle rows of the prefill
  int64_t pos;         // appends: position of the first token (every row)
  // appends in a ragged batch: row b appends row_count[b] (null: n_src)
  // tokens at row_pos[b]; a row whose tokens would end past pos_end is
  // left untouched
  const int64_t* row_pos;
  const int32_t* row_count;
  int64_t pos_end;
  // paged middle (one K group per page): group g of batch row b lives in
  // page block_table[b * pages_per_row + g] of the pool, and the head
  // offsets above are offsets within a page
  uint8_t* pool;
  const int32_t* block_table;
  int64_t page_bytes;
  int32_t pages_per_row;
  int32_t paged;
  int32_t n_kv;
  int32_t n_sink;
  int32_t window;
  int32_t slots;
  int32_t bits;
  int32_t pad;
  QuantHead heads[LEANK_MAX_KV_HEADS];
};

// Where group g (64 middle rows) of batch row b and live head hd lives: its
// K codes, K (scale, min) pairs, first V code block and first V row
// parameters.
struct QGroupAt {
  uint8_t* k_codes;
  float* k_par;
  uint8_t* v_codes;
  float* v_par;
};

__device__ __forceinline__ QGroupAt q_group_at(const QuantParams& p, const QuantHead& hd, int b,
                                               int64_t g) {
  QGroupAt a;
  const int64_t c = hd.kept;
  if (p.paged) {
    uint8_t* base = p.pool + static_cast<int64_t>(p.block_table[static_cast<int64_t>(b) * p.pages_per_row + g]) *
                                 p.page_bytes;
    a.k_codes = base + hd.k_q_off;
    a.k_par = reinterpret_cast<float*>(base) + hd.k_qp_off;
    a.v_codes = base + hd.v_q_off;
    a.v_par = reinterpret_cast<float*>(base) + hd.v_qp_off;
  } else {
    const int64_t blk_bytes = LEANK_HEAD_DIM * LEANK_V_BLOCK * p.bits / 8;
    a.k_codes = p.k_q + hd.k_q_off + (static_cast<int64_t>(b) * p.g_rows + g * LEANK_QUANT_GROUP) * c * p.bits / 8;
    a.k_par = p.k_qp + hd.k_qp_off + (static_cast<int64_t>(b) * (p.g_rows / LEANK_QUANT_GROUP) + g) * c * 2;
    a.v_codes = p.v_q + hd.v_q_off +
                (static_cast<int64_t>(b) * (p.v_rows_cap / LEANK_V_BLOCK) + g * (LEANK_QUANT_GROUP / LEANK_V_BLOCK)) *
                    blk_bytes;
    a.v_par = p.v_qp + hd.v_qp_off + (static_cast<int64_t>(b) * p.mid_cap + g * LEANK_QUANT_GROUP) * 2;
  }
  return a;
}

// ---------------------------------------------------------------- the code decision
//
// A group of values x is held as codes of `bits` bits with lo = min x,
// scale = (max x - lo) / (2^bits - 1), code = rint((x - lo) / scale) clamped
// to [0, 2^bits - 1] (0 when scale = 0), decided in IEEE float32: one
// subtraction, one correctly rounded division, round half to even.

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// scale of a group with minimum lo and maximum hi
__device__ __forceinline__ float quant_scale(float lo, float hi, int bits) {
  return __fdiv_rn(__fsub_rn(hi, lo), static_cast<float>((1 << bits) - 1));
}

__device__ __forceinline__ uint32_t quant_code(float x, float lo, float scale, int bits) {
  if (!(scale > 0.0f)) return 0u;
  const float r = rintf(__fdiv_rn(__fsub_rn(x, lo), scale));
  const float top = static_cast<float>((1 << bits) - 1);
  return static_cast<uint32_t>(fminf(fmaxf(r, 0.0f), top));
}

// One V row (128 channels, a wavefront's 64 lanes holding channels 2 lane,
// 2 lane + 1 as floats x0, x1) quantized per token: the two codes, and the
// row's (scale, lo) in every lane.
__device__ __forceinline__ void quantize_v_row_regs(float x0, float x1, int bits, uint32_t* c0,
                                                    uint32_t* c1, float* scale_out, float* lo_out) {
  float lo = fminf(x0, x1), hi = fmaxf(x0, x1);
  for (int off = 32; off > 0; off >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  const float scale = quant_scale(lo, hi, bits);
  *c0 = quant_code(x0, lo, scale, bits);
  *c1 = quant_code(x1, lo, scale, bits);
  *scale_out = scale;
  *lo_out = lo;
}

// The same, writing (scale, lo) to params through lane 0.
__device__ __forceinline__ void quantize_v_row(float x0, float x1, int bits, float* params,
                                               uint32_t* c0, uint32_t* c1) {
  float scale, lo;
  quantize_v_row_regs(x0, x1, bits, c0, c1, &scale, &lo);
  if ((threadIdx.x & 63) == 0) {
    params[0] = scale;
    params[1] = lo;
  }
}

// Byte offset of (row e of a block, channel ch) within one V code block
// (4-bit: byte k of a channel's 4 bytes holds rows k and k + 4), and the
// nibble of that byte holding row e.
__device__ __forceinline__ int v_code_byte(int ch, int e, int bits) {
  return bits == 8 ? ch * 8 + e : ch * 4 + (e & 3);
}
__device__ __forceinline__ int v_code_shift(int e) { return 4 * (e >> 2); }

__device__ __forceinline__ float group_value(float x) { return x; }
__device__ __forceinline__ float group_value(uint16_t x) { return bf16_to_f32(x); }

// Quantizes one complete K group (64 rows x c kept channels in
// s_x[row * c + j], floats or bf16 bits) per channel into codes (row-major,
// bits wide; 4-bit: the even channel in the low nibble) and (scale, lo)
// pairs [c][2], and leaves each channel's scale and lo in s_scale / s_lo.
// Every thread of a workgroup of `threads` threads calls it.
template <typename T>
__device__ __forceinline__ void quantize_k_group_wg(const T* s_x, int c, int bits, int threads,
                                                    float* s_scale, float* s_lo, uint8_t* codes,
                                                    float* params) {
  const int t = threadIdx.x;
  if (t < c) {
    float lo = group_value(s_x[t]), hi = lo;
    for (int r = 1; r < LEANK_QUANT_GROUP; ++r) {
      lo = fminf(lo, group_value(s_x[r * c + t]));
      hi = fmaxf(hi, group_value(s_x[r * c + t]));
    }
    const float scale = quant_scale(lo, hi, bits);
    s_scale[t] = scale;
    s_lo[t] = lo;
    params[2 * t] = scale;
    params[2 * t + 1] = lo;
  }
  __syncthreads();
  if (bits == 8) {
    for (int i = t; i < LEANK_QUANT_GROUP * c; i += threads) {
      const int j = i % c;
      codes[i] = static_cast<uint8_t>(quant_code(group_value(s_x[i]), s_lo[j], s_scale[j], 8));
    }
  } else {
    for (int i = t; i < LEANK_QUANT_GROUP * c / 2; i += threads) {
      const int j = (2 * i) % c;
      const uint32_t a = quant_code(group_value(s_x[2 * i]), s_lo[j], s_scale[j], 4);
      const uint32_t b = quant_code(group_value(s_x[2 * i + 1]), s_lo[j + 1], s_scale[j + 1], 4);
      codes[i] = static_cast<uint8_t>(a | (b << 4));
    }
  }
}

void fill_quant_params(const leank_layer_cache* c, QuantParams* p);
// Middle rows of a prefill of n_new tokens into an empty cache (the sink and
// window rows are written by the ordinary pack kernel).
int quant_pack_bulk(const leank_layer_cache* c, const void* k_new, const void* v_new,
                    int64_t n_new, hipStream_t s);
// n_new tokens at positions pos0 .. (every row), or, with row_pos set, a
// ragged append as in leank_pack_k_rows (tokens ending past pos_end leave
// the row untouched): ring and middle, one token after the other.
int quant_append(const leank_layer_cache* c, const void* k_new, const void* v_new, int64_t pos0,
                 int64_t n_new, const int64_t* row_pos, const int32_t* row_count, int64_t pos_end,
                 hipStream_t s);

}  // namespace leank
