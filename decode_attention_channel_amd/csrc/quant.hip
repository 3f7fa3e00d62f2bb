// Low-bit middle streams: packing into a cache planned by
// leank_plan_layer_q (LeanK page, section 4.2 and its deployment notes --
// quantization after prune and reorganisation; white paper section 5.2.1 --
// KIVI's per-channel K and per-token V).  The code decision is in quant.h.
// K: per kept channel over each group of 64 middle rows; the rows of a group
// that is not complete yet wait in a bf16 staging buffer.  V: per token.

#include "quant.h"

namespace leank {
namespace {

constexpr int kQThreads = 256;


__device__ __forceinline__ void quantize_k_group(const float* s_x, int c, int bits, float* s_scale,
                                                 float* s_lo, uint8_t* codes, float* params) {
  quantize_k_group_wg(s_x, c, bits, kQThreads, s_scale, s_lo, codes, params);
}

// ---------------------------------------------------------------- bulk prefill

// Grid: batch x n_kv x groups.  Group g of a live head's middle: complete
// groups are quantized, the incomplete one goes to staging.  Middle row r
// is token n_sink + r of the source.
__global__ __launch_bounds__(kQThreads) void quant_k_bulk_kernel(const QuantParams p) {
  __shared__ float s_x[LEANK_QUANT_GROUP * LEANK_HEAD_DIM];
  __shared__ float s_scale[LEANK_HEAD_DIM];
  __shared__ float s_lo[LEANK_HEAD_DIM];
  __shared__ int16_t s_idx[LEANK_HEAD_DIM];
  const int64_t n_groups = (p.t_mid + LEANK_QUANT_GROUP - 1) / LEANK_QUANT_GROUP;
  const int64_t g = blockIdx.x % n_groups;
  const int64_t pair = blockIdx.x / n_groups;
  const int b = static_cast<int>(pair / p.n_kv);
  const int h = static_cast<int>(pair % p.n_kv);
  const QuantHead hd = p.heads[h];
  const int c = hd.kept;
  if (c <= 0) return;  // dead head: no middle
  const int t = threadIdx.x;
  if (t < LEANK_HEAD_DIM) s_idx[t] = p.kept_idx[h * LEANK_HEAD_DIM + t] & (LEANK_HEAD_DIM - 1);
  __syncthreads();
  const int64_t r0 = g * LEANK_QUANT_GROUP;
  const int rows = static_cast<int>(min<int64_t>(LEANK_QUANT_GROUP, p.t_mid - r0));
  const uint16_t* src = p.k_src + (pair * p.n_src + p.n_sink + r0) * LEANK_HEAD_DIM;
  if (rows < LEANK_QUANT_GROUP) {
    // incomplete group: bf16 rows to staging row r % 64
    uint16_t* stage = p.k_stage + hd.k_stage_off + static_cast<int64_t>(b) * LEANK_QUANT_GROUP * c;
    for (int i = t; i < rows * c; i += kQThreads) {
      const int r = i / c, j = i - (i / c) * c;
      stage[i] = src[static_cast<int64_t>(r) * LEANK_HEAD_DIM + s_idx[j]];
    }
    return;
  }
  for (int i = t; i < LEANK_QUANT_GROUP * c; i += kQThreads) {
    const int r = i / c, j = i - (i / c) * c;
    s_x[i] = bf16_to_f32(src[static_cast<int64_t>(r) * LEANK_HEAD_DIM + s_idx[j]]);
  }
  __syncthreads();
  const QGroupAt at = q_group_at(p, hd, b, g);
  quantize_k_group(s_x, c, p.bits, s_scale, s_lo, at.k_codes, at.k_par);
}

// Grid: batch x n_kv x ceil(t_mid / 8).  One 8-row V block per workgroup:
// each wavefront quantizes two rows (per token), the block is written whole.
__global__ __launch_bounds__(kQThreads) void quant_v_bulk_kernel(const QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_blk[LEANK_HEAD_DIM * LEANK_V_BLOCK];
  const int64_t n_blocks = (p.t_mid + LEANK_V_BLOCK - 1) / LEANK_V_BLOCK;
  const int64_t blk = blockIdx.x % n_blocks;
  const int64_t pair = blockIdx.x / n_blocks;
  const int b = static_cast<int>(pair / p.n_kv);
  const int h = static_cast<int>(pair % p.n_kv);
  const QuantHead hd = p.heads[h];
  if (hd.kept <= 0) return;  // dead head: no middle V
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int blk_bytes = LEANK_HEAD_DIM * LEANK_V_BLOCK * p.bits / 8;
  for (int i = t; i < blk_bytes; i += kQThreads) s_blk[i] = 0;
  __syncthreads();
  for (int e = t >> 6; e < LEANK_V_BLOCK; e += kQThreads / 64) {
    const int64_t r = blk * LEANK_V_BLOCK + e;
    if (r >= p.t_mid) break;  // wavefront-uniform
    const uint32_t w = reinterpret_cast<const uint32_t*>(
        p.v_src + (pair * p.n_src + p.n_sink + r) * LEANK_HEAD_DIM)[lane];
    uint32_t c0, c1;
    quantize_v_row(bf16_lo(w), bf16_hi(w), p.bits,
                   q_group_at(p, hd, b, r / LEANK_QUANT_GROUP).v_par + (r % LEANK_QUANT_GROUP) * 2, &c0, &c1);
    if (p.bits == 8) {
      s_blk[v_code_byte(2 * lane, e, 8)] = static_cast<uint8_t>(c0);
      s_blk[v_code_byte(2 * lane + 1, e, 8)] = static_cast<uint8_t>(c1);
    } else {
      // rows k and k + 4 share a byte and are quantized by different
      // wavefronts: combine the nibbles with LDS atomic ors
      atomicOr(reinterpret_cast<uint32_t*>(s_blk) + v_code_byte(2 * lane, e, 4) / 4,
               c0 << (8 * (v_code_byte(2 * lane, e, 4) % 4) + v_code_shift(e)));
      atomicOr(reinterpret_cast<uint32_t*>(s_blk) + v_code_byte(2 * lane + 1, e, 4) / 4,
               c1 << (8 * (v_code_byte(2 * lane + 1, e, 4) % 4) + v_code_shift(e)));
    }
  }
  __syncthreads();
  constexpr int kBlocksPerGroup = LEANK_QUANT_GROUP / LEANK_V_BLOCK;
  uint8_t* dst = q_group_at(p, hd, b, blk / kBlocksPerGroup).v_codes + (blk % kBlocksPerGroup) * blk_bytes;
  for (int i = t; i < blk_bytes / 16; i += kQThreads)
    reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(s_blk)[i];
}

// ---------------------------------------------------------------- one token

// Grid: batch x n_kv.  Appends the token at position p.pos: a sink or ring
// row for the new token; the token leaving the window (or, with no window,
// the new token) becomes middle row r: K kept channels to staging row
// r % 64, V quantized per token into its block (read, one row replaced,
// written whole); when r completes its group, the group is quantized.
__global__ __launch_bounds__(kQThreads) void quant_append_kernel(const QuantParams p) {
  __shared__ float s_x[LEANK_QUANT_GROUP * LEANK_HEAD_DIM];
  __shared__ float s_scale[LEANK_HEAD_DIM];
  __shared__ float s_lo[LEANK_HEAD_DIM];
  __shared__ int16_t s_idx[LEANK_HEAD_DIM];
  __shared__ __attribute__((aligned(16))) uint16_t s_tok[2][LEANK_HEAD_DIM];  // middle token K, V
  __shared__ __attribute__((aligned(16))) uint8_t s_blk[LEANK_HEAD_DIM * LEANK_V_BLOCK];
  const int64_t pair = blockIdx.x;
  const int b = static_cast<int>(pair / p.n_kv);
  const int h = static_cast<int>(pair % p.n_kv);
  const QuantHead hd = p.heads[h];
  const int c = hd.kept;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int S = p.n_sink, W = p.window;
  uint16_t* ring_k = p.k_sl + pair * p.slots * LEANK_HEAD_DIM;
  uint16_t* ring_v = p.v_sl + pair * p.v_sl_rows * LEANK_HEAD_DIM;
  int64_t pos0 = p.pos, count = p.n_src;
  if (p.row_pos) {
    pos0 = p.row_pos[b];
    count = p.row_count ? p.row_count[b] : p.n_src;
    // a row whose tokens fall outside the cache is left untouched
    if (pos0 < 0 || count < 0 || count > p.n_src || pos0 + count > p.pos_end) return;
  }
  for (int64_t u = 0; u < count; ++u) {
    // tokens in order: the previous token's reads and writes (ring row, V
    // block, staged K row) are done and visible to the whole workgroup
    if (u > 0) __syncthreads();
    const int64_t pos = pos0 + u;
    const uint16_t* k_new = p.k_src + (pair * p.n_src + u) * LEANK_HEAD_DIM;
    const uint16_t* v_new = p.v_src + (pair * p.n_src + u) * LEANK_HEAD_DIM;
    const int slot = pos < S ? static_cast<int>(pos) : (W > 0 ? S + static_cast<int>((pos - S) % W) : -1);

    // the token that becomes a middle row, if any
    int64_t r = -1;
    if (c > 0) {
      if (pos >= S && W == 0) r = pos - S;
      else if (W > 0 && pos - W >= S) r = pos - W - S;
    }
    if (t < LEANK_HEAD_DIM) {
      s_idx[t] = p.kept_idx[h * LEANK_HEAD_DIM + t] & (LEANK_HEAD_DIM - 1);
      if (r >= 0) {
        const bool from_ring = W > 0;
        s_tok[0][t] = from_ring ? ring_k[slot * LEANK_HEAD_DIM + t] : k_new[t];
        s_tok[1][t] = from_ring ? ring_v[v_elem(slot, t)] : v_new[t];
      }
    }
    const int blk_bytes = LEANK_HEAD_DIM * LEANK_V_BLOCK * p.bits / 8;
    uint8_t* vblk = nullptr;
    if (r >= 0) {
      vblk = q_group_at(p, hd, b, r / LEANK_QUANT_GROUP).v_codes +
             ((r % LEANK_QUANT_GROUP) / LEANK_V_BLOCK) * blk_bytes;
      for (int i = t; i < blk_bytes / 16; i += kQThreads)
        reinterpret_cast<uint4*>(s_blk)[i] = reinterpret_cast<const uint4*>(vblk)[i];
    }
    __syncthreads();  // the ring row is read before it is replaced below

    if (slot >= 0 && t < 64) {
      // the new token to its sink or ring row
      reinterpret_cast<uint32_t*>(ring_k + slot * LEANK_HEAD_DIM)[t] =
          reinterpret_cast<const uint32_t*>(k_new)[t];
      store_v_row_word(ring_v, slot, t, reinterpret_cast<const uint32_t*>(v_new)[t]);
    }
    if (r < 0) continue;

    const int e = static_cast<int>(r % LEANK_V_BLOCK);
    const int in_group = static_cast<int>(r % LEANK_QUANT_GROUP);
    if (t < 64) {
      // V of the middle row, quantized per token, replaces row e of its block
      const uint32_t w = reinterpret_cast<const uint32_t*>(s_tok[1])[lane];
      uint32_t c0, c1;
      quantize_v_row(bf16_lo(w), bf16_hi(w), p.bits,
                     q_group_at(p, hd, b, r / LEANK_QUANT_GROUP).v_par + (r % LEANK_QUANT_GROUP) * 2, &c0, &c1);
  #pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ch = 2 * lane + u;
        const uint32_t code = u ? c1 : c0;
        const int at = v_code_byte(ch, e, p.bits);
        if (p.bits == 8) {
          s_blk[at] = static_cast<uint8_t>(code);
        } else {
          const int sh = v_code_shift(e);
          s_blk[at] = static_cast<uint8_t>((s_blk[at] & ~(0xF << sh)) | (code << sh));
        }
      }
    } else if (t >= 64 && t - 64 < c) {
      // K kept channels to staging
      const int j = t - 64;
      p.k_stage[hd.k_stage_off + (static_cast<int64_t>(b) * LEANK_QUANT_GROUP + in_group) * c + j] =
          s_tok[0][s_idx[j]];
    }
    __syncthreads();
    for (int i = t; i < blk_bytes / 16; i += kQThreads)
      reinterpret_cast<uint4*>(vblk)[i] = reinterpret_cast<const uint4*>(s_blk)[i];

    if (in_group != LEANK_QUANT_GROUP - 1) continue;
    // the row completes its group: quantize the 64 staged rows (this row from LDS)
    const uint16_t* stage = p.k_stage + hd.k_stage_off + static_cast<int64_t>(b) * LEANK_QUANT_GROUP * c;
    for (int i = t; i < LEANK_QUANT_GROUP * c; i += kQThreads) {
      const int row = i / c, j = i - (i / c) * c;
      s_x[i] = bf16_to_f32(row == LEANK_QUANT_GROUP - 1 ? s_tok[0][s_idx[j]] : stage[i]);
    }
    __syncthreads();
    const QGroupAt at = q_group_at(p, hd, b, r / LEANK_QUANT_GROUP);
    quantize_k_group(s_x, c, p.bits, s_scale, s_lo, at.k_codes, at.k_par);
  }
}

}  // namespace

void fill_quant_params(const leank_layer_cache* c, QuantParams* p) {
  memset(p, 0, sizeof(*p));
  p->k_q = static_cast<uint8_t*>(c->k_q);
  p->k_qp = static_cast<float*>(c->k_qp);
  p->k_stage = static_cast<uint16_t*>(c->k_stage);
  p->v_q = static_cast<uint8_t*>(c->v_q);
  p->v_qp = static_cast<float*>(c->v_qp);
  p->k_sl = static_cast<uint16_t*>(c->k_sl);
  p->v_sl = static_cast<uint16_t*>(c->v_sl);
  p->kept_idx = c->kept_idx;
  p->mid_cap = c->mid_capacity;
  p->g_rows = (c->mid_capacity + LEANK_QUANT_GROUP - 1) / LEANK_QUANT_GROUP * LEANK_QUANT_GROUP;
  p->v_rows_cap = v_rows(c->mid_capacity);
  p->v_sl_rows = v_rows(static_cast<int64_t>(c->n_sink) + c->window);
  p->n_kv = c->n_kv_heads;
  p->n_sink = c->n_sink;
  p->window = c->window;
  p->slots = c->n_sink + c->window;
  p->bits = c->quant_bits;
  p->paged = c->page_rows != 0;
  p->pool = static_cast<uint8_t*>(c->pool);
  p->block_table = c->block_table;
  p->page_bytes = static_cast<int64_t>(c->page_bytes);
  p->pages_per_row = c->pages_per_row;
  for (int h = 0; h < c->n_kv_heads; ++h) {
    p->heads[h].kept = c->kept_count[h];
    p->heads[h].k_q_off = c->k_q_off[h];
    p->heads[h].k_qp_off = c->k_qp_off[h];
    p->heads[h].k_stage_off = c->k_stage_off[h];
    p->heads[h].v_q_off = c->v_q_off[h];
    p->heads[h].v_qp_off = c->v_qp_off[h];
  }
}

int quant_pack_bulk(const leank_layer_cache* c, const void* k_new, const void* v_new,
                    int64_t n_new, hipStream_t s) {
  const int64_t t_mid = std::max<int64_t>(0, n_new - c->n_sink - c->window);
  if (t_mid == 0 || c->n_live == 0) return LEANK_OK;
  QuantParams p;
  fill_quant_params(c, &p);
  p.k_src = static_cast<const uint16_t*>(k_new);
  p.v_src = static_cast<const uint16_t*>(v_new);
  p.n_src = n_new;
  p.t_mid = t_mid;
  const int64_t pairs = static_cast<int64_t>(c->batch) * c->n_kv_heads;
  const int64_t k_blocks = pairs * ((t_mid + LEANK_QUANT_GROUP - 1) / LEANK_QUANT_GROUP);
  const int64_t v_blocks = pairs * ((t_mid + LEANK_V_BLOCK - 1) / LEANK_V_BLOCK);
  if (k_blocks > INT32_MAX || v_blocks > INT32_MAX) return LEANK_EUNSUPPORTED;
  hipLaunchKernelGGL(quant_k_bulk_kernel, dim3(static_cast<unsigned>(k_blocks)), dim3(kQThreads),
                     0, s, p);
  LEANK_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(quant_v_bulk_kernel, dim3(static_cast<unsigned>(v_blocks)), dim3(kQThreads),
                     0, s, p);
  LEANK_HIP_TRY(hipGetLastError());
  return LEANK_OK;
}

int quant_append(const leank_layer_cache* c, const void* k_new, const void* v_new, int64_t pos0,
                 int64_t n_new, const int64_t* row_pos, const int32_t* row_count, int64_t pos_end,
                 hipStream_t s) {
  QuantParams p;
  fill_quant_params(c, &p);
  p.k_src = static_cast<const uint16_t*>(k_new);
  p.v_src = static_cast<const uint16_t*>(v_new);
  p.n_src = n_new;
  p.pos = pos0;
  p.row_pos = row_pos;
  p.row_count = row_count;
  p.pos_end = pos_end;
  const int64_t pairs = static_cast<int64_t>(c->batch) * c->n_kv_heads;
  if (pairs > INT32_MAX) return LEANK_EUNSUPPORTED;
  hipLaunchKernelGGL(quant_append_kernel, dim3(static_cast<unsigned>(pairs)), dim3(kQThreads), 0,
                     s, p);
  LEANK_HIP_TRY(hipGetLastError());
  return LEANK_OK;
}

}  // namespace leank
