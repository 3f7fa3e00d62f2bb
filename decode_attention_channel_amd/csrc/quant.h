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
  int64_t pos;         // one token: its position
  int32_t n_kv;
  int32_t n_sink;
  int32_t window;
  int32_t slots;
  int32_t bits;
  int32_t pad;
  QuantHead heads[LEANK_MAX_KV_HEADS];
};

void fill_quant_params(const leank_layer_cache* c, QuantParams* p);
// Middle rows of a prefill of n_new tokens into an empty cache (the sink and
// window rows are written by the ordinary pack kernel).
int quant_pack_bulk(const leank_layer_cache* c, const void* k_new, const void* v_new,
                    int64_t n_new, hipStream_t s);
// One token at position pos, ring and middle.
int quant_append_one(const leank_layer_cache* c, const void* k_new, const void* v_new, int64_t pos,
                     hipStream_t s);

}  // namespace leank
