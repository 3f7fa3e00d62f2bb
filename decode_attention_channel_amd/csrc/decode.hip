// Host entry points of the decode path: leank_decode_attn and its ragged
// form, the fused decode step (append + attention in the same two kernels)
// and its ragged form, and leank_workspace_init.  The kernels live in
// decode_kernels.h, instantiated per group size in decode_g1.hip ..
// decode_g8.hip.

#include <mutex>

#include "decode_kernels.h"
#include "quant.h"

// Scratch of leank_decode_step_noalloc: the split-K records of one call, in
// a file-scope device array instead of a caller's workspace.  Each device
// the library runs on holds its own copy until the process ends.  Host code
// never uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[LEANK_NOALLOC_SCRATCH_BYTES];

namespace leank {

#define LEANK_EXTERN_DECODE(G)                                                              \
  extern template int launch_decode<G, 0>(const DecodeParams&, int64_t, int64_t, int, hipStream_t); \
  extern template int launch_decode<G, 4>(const DecodeParams&, int64_t, int64_t, int, hipStream_t); \
  extern template int launch_decode<G, 8>(const DecodeParams&, int64_t, int64_t, int, hipStream_t);
LEANK_EXTERN_DECODE(1)
LEANK_EXTERN_DECODE(2)
LEANK_EXTERN_DECODE(3)
LEANK_EXTERN_DECODE(4)
LEANK_EXTERN_DECODE(5)
LEANK_EXTERN_DECODE(6)
LEANK_EXTERN_DECODE(7)
LEANK_EXTERN_DECODE(8)
#undef LEANK_EXTERN_DECODE

namespace {

// The low-bit segments must follow the canonical layout of
// leank_plan_layer_q (the kernels derive them from the kept-channel prefix
// and the live rank of each head).
bool canonical_quant_layout(const leank_layer_cache* c, int64_t* c_prefix, int64_t* rank) {
  const int64_t batch = c->batch, bits = c->quant_bits;
  const int64_t groups = (c->mid_capacity + LEANK_QUANT_GROUP - 1) / LEANK_QUANT_GROUP;
  const int64_t g_rows = groups * LEANK_QUANT_GROUP;
  const bool paged = c->page_rows != 0;  // in-page offsets, checked by validate_cache
  int64_t pre = 0, n = 0;
  for (int i = 0; i < c->n_kv_heads; ++i) {
    const int h = c->group_order[i];
    const int64_t kept = c->kept_count[h];
    if (h < 0 || h >= c->n_kv_heads) return false;
    if (kept <= 0) continue;
    if (!paged &&
        (c->k_q_off[h] != batch * g_rows * pre * bits / 8 || c->k_qp_off[h] != batch * groups * pre * 2 ||
         c->k_stage_off[h] != batch * LEANK_QUANT_GROUP * pre ||
         c->v_q_off[h] != n * batch * v_rows(c->mid_capacity) * LEANK_HEAD_DIM * bits / 8 ||
         c->v_qp_off[h] != n * batch * c->mid_capacity * 2))
      return false;
    c_prefix[h] = pre;
    rank[h] = n;
    pre += kept;
    ++n;
  }
  return true;
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n_words) {
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; k < n_words;
       k += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[k] = 0u;
}

}  // namespace
}  // namespace leank

using namespace leank;

extern "C" int leank_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes % 4) return LEANK_EINVAL;
  const int64_t words = static_cast<int64_t>(workspace_bytes / 4);
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 4096);
  if (blocks == 0) return LEANK_OK;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(workspace), words);
  LEANK_HIP_TRY(hipGetLastError());
  return LEANK_OK;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the current device, looked up on the
// first call on that device (with it current) and kept.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LEANK_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return LEANK_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LEANK_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LEANK_OK;
}

}  // namespace


namespace {

// What a call adds to plain decode attention over the cached rows.
struct CallExtras {
  const int32_t* ctx_lens = nullptr;  // ragged decode: per-row lengths
  bool step = false;                  // fused step: append one token, then attend
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int64_t* row_pos = nullptr;   // ragged step: per-row positions
  bool scratch = false;               // records in the library's device scratch, not a workspace
};

// plan_len: rows the regular items cover -- the context length of a decode
// call, the rows cached before the append in a step (whose context is one
// more).
int decode_impl(const leank_layer_cache* c, const void* q, const CallExtras& x, int64_t plan_len,
                float scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_cache(c, true);
  if (st != LEANK_OK) return st;
  const bool quant = c->quant_bits != 0;
  int64_t q_prefix[LEANK_MAX_KV_HEADS] = {0}, q_rank[LEANK_MAX_KV_HEADS] = {0};
  if (quant && !canonical_quant_layout(c, q_prefix, q_rank)) return LEANK_EINVAL;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return LEANK_EINVAL;
  if (x.step) {
    if (!x.k_new || !x.v_new || !aligned16(x.k_new) || !aligned16(x.v_new)) return LEANK_EINVAL;
    if (plan_len < 0) return LEANK_EINVAL;
    if (plan_len + 1 > c->max_ctx) return LEANK_ECAPACITY;
  } else {
    if (plan_len < 1) return LEANK_EINVAL;
    if (plan_len > c->max_ctx) return LEANK_ECAPACITY;
  }
  if (!(scale > 0.0f) || !isfinite(scale)) return LEANK_EINVAL;
  if (x.scratch) {  // every argument is checked: look the device scratch up
    st = scratch_ptr(&workspace);
    if (st != LEANK_OK) return st;
    workspace_bytes = LEANK_NOALLOC_SCRATCH_BYTES;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool step = x.step;
  bool lens_from_pos = false;  // attention over row_pos[b] + 1 tokens after a separate append
  if (quant && step) {
    // the middle row this append writes (every live head writes the same
    // row); when it completes a K group, every row of that group changes to
    // codes, which the other items of a fused call would still read staged:
    // such a step runs the append kernel, then the attention over pos + 1.
    // So does every ragged step, whose rows complete groups at different
    // steps.
    const int64_t pos = plan_len;
    const int64_t r = c->window > 0 ? pos - c->window - c->n_sink : pos - c->n_sink;
    if (x.row_pos || (r >= 0 && r % LEANK_QUANT_GROUP == LEANK_QUANT_GROUP - 1)) {
      WorkPlan wq;
      make_work_plan(c, plan_len + 1, 0, &wq);
      if (!workspace || !aligned16(workspace) || workspace_bytes < wq.workspace_bytes)
        return LEANK_EWORKSPACE;
      st = x.row_pos ? quant_append(c, x.k_new, x.v_new, 0, 1, x.row_pos, nullptr, plan_len + 1, s)
                     : quant_append(c, x.k_new, x.v_new, pos, 1, nullptr, nullptr, c->max_ctx, s);
      if (st != LEANK_OK) return st;
      step = false;
      lens_from_pos = x.row_pos != nullptr;
      plan_len += 1;
    }
  }
  WorkPlan w;
  make_work_plan(c, plan_len, step ? 1 : 0, &w);
  if (!workspace || !aligned16(workspace) || workspace_bytes < w.workspace_bytes)
    return LEANK_EWORKSPACE;
  if (w.n_items > INT32_MAX) return LEANK_EUNSUPPORTED;

  DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(q);
  p.k_sl = static_cast<const uint16_t*>(c->k_sl);
  p.v_sl = static_cast<const uint16_t*>(c->v_sl);
  p.k_prun = static_cast<const uint16_t*>(c->k_prun);
  p.v_mid = static_cast<const uint16_t*>(c->v_mid);
  p.kept_idx = c->kept_idx;
  p.out = out;
  p.ctx_lens = x.ctx_lens;
  p.k_new = static_cast<const uint16_t*>(x.k_new);
  p.v_new = static_cast<const uint16_t*>(x.v_new);
  p.row_pos = x.row_pos;
  p.step_pos = plan_len;
  p.step = w.step;
  p.lens_from_pos = lens_from_pos ? 1 : 0;
  p.n_sink = c->n_sink;
  p.window = c->window;
  p.max_len = static_cast<int32_t>(plan_len);
  p.partials = static_cast<float*>(workspace);
  p.mid_cap = c->mid_capacity;
  p.v_mid_rows = v_rows(c->mid_capacity);
  p.v_sl_rows = v_rows(static_cast<int64_t>(c->n_sink) + c->window);
  p.n_kv = c->n_kv_heads;
  p.n_q = c->n_q_heads;
  p.slots = c->n_sink + c->window;
  p.t_sl = w.t_sl;
  p.t_mid = w.t_mid;
  p.n_sl_items = w.n_sl_items;
  p.sl_rows = w.sl_rows;
  p.items_per_b = w.items_per_b;
  p.bulk_per_b = w.bulk_per_b;
  p.tail_per_b = w.tail_per_b;
  p.n_bulk = static_cast<int64_t>(w.bulk_per_b) * c->batch;
  p.n_sl_all = w.sl_first ? static_cast<int64_t>(c->batch) * c->n_kv_heads * w.n_sl_items : 0;
  {
    int32_t be = 0, te = 0;
    for (int h = 0; h < 8; ++h) {
      if (h < c->n_kv_heads - 1) {
        be += (w.sl_first ? 0 : w.n_sl_items) + w.n_mid_b[h];
        te += w.n_mid[h] - w.n_mid_b[h];
        p.bulk_end8[h] = be;
        p.tail_end8[h] = te;
      } else {
        p.bulk_end8[h] = INT32_MAX;
        p.tail_end8[h] = INT32_MAX;
      }
    }
  }
  p.partial_stride = w.partial_stride;
  // pairs with many items get their channels split over several combine workgroups
  int32_t max_items = 0;
  for (int h = 0; h < c->n_kv_heads; ++h)
    max_items = std::max(max_items, w.n_sl_items + w.n_mid[h]);
#ifndef LEANK_COMBINE_WAVE
#define LEANK_COMBINE_WAVE 1
#endif
  // channel slices per (pair, query head): 8 * slices item groups per
  // workgroup, with up to LEANK_COMBINE_SLICE_ITEMS items per slice, so
  // that each thread merges up to 8 items (32 slices at most: one float4 of
  // channels per workgroup).  Measured on the 128K-token layer at batch 1
  // (412 items in its one live pair): 16 / 32 / 64 / 128 / 256 items per
  // slice gave 22.6 / 21.3 / 21.0 / 21.6 / 22.6 us per step.
#ifndef LEANK_COMBINE_SLICE_ITEMS
#define LEANK_COMBINE_SLICE_ITEMS 64
#endif
  int slices = 1;
  while (slices < 32 && LEANK_COMBINE_SLICE_ITEMS * slices < max_items) slices *= 2;
  p.combine_slices = slices;
  // few items per pair: one wavefront per (pair, head) merges them without
  // barriers (measured faster up to 32 items)
  if (LEANK_COMBINE_WAVE && max_items <= kWaveCombineItems) p.combine_slices = 0;
  p.wave_items = max_items;
  p.qk_scale = scale * kLog2e;
  p.n_batch = c->batch;
  p.paged = c->page_rows != 0;
  p.pool = static_cast<const uint16_t*>(c->pool);
  p.block_table = c->block_table;
  p.page_elems = static_cast<int64_t>(c->page_bytes / 2);
  p.pages_per_row = c->pages_per_row;
  if (quant) {
    p.k_q = static_cast<const uint8_t*>(c->k_q);
    p.k_qp = static_cast<const float*>(c->k_qp);
    p.k_stage = static_cast<const uint16_t*>(c->k_stage);
    p.v_q = static_cast<const uint8_t*>(c->v_q);
    p.v_qp = static_cast<const float*>(c->v_qp);
    p.q_groups = (c->mid_capacity + LEANK_QUANT_GROUP - 1) / LEANK_QUANT_GROUP;
  }
  for (int h = 0; h < c->n_kv_heads; ++h) {
    p.heads[h].k_off = quant ? q_prefix[h] : c->k_prun_off[h];
    p.heads[h].v_off = quant ? q_rank[h] : c->v_mid_off[h];
    p.heads[h].kept = c->kept_count[h];
    p.heads[h].n_mid = w.n_mid[h];
    p.heads[h].mid_rows = w.mid_rows[h];
    p.heads[h].base = w.head_base[h];
    p.heads[h].n_mid_b = w.n_mid_b[h];
    p.heads[h].mid_rows_t = w.mid_rows_t[h];
    if (quant && p.paged && c->kept_count[h] > 0) {
      p.heads[h].pq_k_codes = static_cast<int32_t>(c->k_q_off[h]);
      p.heads[h].pq_k_par = static_cast<int32_t>(4 * c->k_qp_off[h]);
      p.heads[h].pq_v_codes = static_cast<int32_t>(c->v_q_off[h]);
      p.heads[h].pq_v_par = static_cast<int32_t>(4 * c->v_qp_off[h]);
    }
  }
  const int64_t n_pairs = static_cast<int64_t>(c->batch) * c->n_kv_heads;
  const int qb = c->quant_bits;
  int kb_max = 1;
  for (int h = 0; h < c->n_kv_heads; ++h) kb_max = std::max(kb_max, (c->kept_count[h] + 31) / 32);
#define LEANK_DISPATCH(G)                                                  \
  case G:                                                                  \
    return qb == 8   ? launch_decode<G, 8>(p, w.n_items, n_pairs, kb_max, s)  \
           : qb == 4 ? launch_decode<G, 4>(p, w.n_items, n_pairs, kb_max, s)  \
                     : launch_decode<G, 0>(p, w.n_items, n_pairs, kb_max, s);
  switch (w.group) {
    LEANK_DISPATCH(1)
    LEANK_DISPATCH(2)
    LEANK_DISPATCH(3)
    LEANK_DISPATCH(4)
    LEANK_DISPATCH(5)
    LEANK_DISPATCH(6)
    LEANK_DISPATCH(7)
    LEANK_DISPATCH(8)
    default: return LEANK_EUNSUPPORTED;
  }
#undef LEANK_DISPATCH
}

}  // namespace

extern "C" int leank_decode_attn(const leank_layer_cache* c, const void* q, int64_t ctx_len,
                                 float scale, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return decode_impl(c, q, CallExtras{}, ctx_len, scale, out, workspace, workspace_bytes, stream);
}

extern "C" int leank_decode_attn_rows(const leank_layer_cache* c, const void* q,
                                      const int32_t* ctx_lens, int64_t max_ctx_len, float scale,
                                      float* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!ctx_lens) return LEANK_EINVAL;
  CallExtras x;
  x.ctx_lens = ctx_lens;
  return decode_impl(c, q, x, max_ctx_len, scale, out, workspace, workspace_bytes, stream);
}

extern "C" int leank_decode_step(const leank_layer_cache* c, const void* q, const void* k_new,
                                 const void* v_new, int64_t pos, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  CallExtras x;
  x.step = true;
  x.k_new = k_new;
  x.v_new = v_new;
  return decode_impl(c, q, x, pos, scale, out, workspace, workspace_bytes, stream);
}

extern "C" int leank_decode_step_rows(const leank_layer_cache* c, const void* q,
                                      const void* k_new, const void* v_new,
                                      const int64_t* row_pos, int64_t max_ctx_len, float scale,
                                      float* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!row_pos || max_ctx_len < 1) return LEANK_EINVAL;
  CallExtras x;
  x.step = true;
  x.k_new = k_new;
  x.v_new = v_new;
  x.row_pos = row_pos;
  return decode_impl(c, q, x, max_ctx_len - 1, scale, out, workspace, workspace_bytes, stream);
}

extern "C" int leank_decode_step_noalloc(const leank_layer_cache* c, const void* q,
                                         const void* k_new, const void* v_new, int64_t pos,
                                         float scale, float* out, void* stream) {
  CallExtras x;
  x.step = true;
  x.k_new = k_new;
  x.v_new = v_new;
  x.scratch = true;
  // the kernels write every record they read, so the scratch needs no clearing
  return decode_impl(c, q, x, pos, scale, out, nullptr, 0, stream);
}
