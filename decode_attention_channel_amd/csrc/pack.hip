// leank_pack_k: route appended tokens into the channel-pruned cache
// (LeanK page, section 3.1 item 2; section 3.2 for heads without middle V).
//
// One wavefront handles one (batch row, KV head, token) unit and moves one
// 256-byte K row and one V row: lane l carries channels 2l, 2l+1.  K rows
// are row-major; V rows live in 8-row blocks (element (r, c) of a region at
// ((r / 8) * 128 + c) * 8 + r % 8), so a lane writes its two V values
// 16 bytes apart.  The kept-channel gather into K_prun reads the source
// word of each kept channel from the lane that holds it (ds_bpermute).

#include "quant.h"

namespace leank {
namespace {

enum PackMode : int32_t {
  kFused = 0,    // n_new <= window: each unit migrates the token its ring row holds, then writes
  kMigrate = 1,  // move window tokens that leave the window to the middle
  kPlace = 2,    // route new tokens to sink rows, the middle or ring rows
};

struct PackHead {
  int64_t k_off;  // elements
  int64_t v_off;  // elements
  int32_t kept;
  int32_t pad;
};

struct PackParams {
  const uint32_t* k_new;
  const uint32_t* v_new;
  uint32_t* k_sl;
  uint16_t* v_sl;
  uint32_t* k_prun;
  uint16_t* v_mid;
  const int16_t* kept_idx;
  int32_t ring_only;   // low-bit cache: middle rows are written by the quantizing kernels
  int32_t paged;       // middle rows in pages through block_table (heads' k_off / v_off are in-page)
  uint16_t* pool;
  const int32_t* block_table;
  int64_t page_elems;
  int64_t pages_per_row;
  int64_t t_old;       // tokens in the cache before the append
  int64_t t_new;       // tokens after it
  int64_t n_new;
  int64_t mid_cap;
  int64_t v_mid_rows;  // stored V rows per batch row of a middle segment (multiple of 8)
  int64_t v_sl_rows;   // stored V rows per (batch row, head) of the ring (multiple of 8)
  int64_t unit_lo;     // kMigrate: position of unit 0
  int64_t units_per_pair;
  int64_t n_units;
  int64_t max_ctx;
  const int64_t* row_pos;    // per-row append position (ragged batches), or null
  const int32_t* row_count;  // per-row token count (ragged batches), or null = n_new
  int32_t n_kv;
  int32_t n_sink;
  int32_t window;
  int32_t slots;
  int32_t mode;
  int32_t pad;
  PackHead heads[LEANK_MAX_KV_HEADS];
};

constexpr int kWordsPerRow = LEANK_HEAD_DIM / 2;  // 64 words of two bf16
// one unit (a wavefront) per workgroup: a one-token append of 512 (batch
// row, head) pairs then spreads over every compute unit (measured: the
// unfused Llama batch-64 step 117.1 -> 116.7 us, Qwen 100.1 -> 99.4 us
// against four units per workgroup)
#ifndef LEANK_PACK_UNITS
#define LEANK_PACK_UNITS 1
#endif
constexpr int kUnitsPerBlock = LEANK_PACK_UNITS;

// Writes one token's K (kept channels) and V (live heads) to middle row r.
__device__ __forceinline__ void write_middle(const PackParams& p, int b, int h, int64_t r,
                                             uint32_t kw, uint32_t vw, int lane) {
  const PackHead hd = p.heads[h];
  if (hd.kept <= 0) return;  // fully pruned head: no middle K, no middle V
  const int j0 = 2 * lane;
  // channel ids are masked into [0, 128) so that bad ids cannot leave the row
  const int c0 = j0 < hd.kept ? (p.kept_idx[h * LEANK_HEAD_DIM + j0] & (LEANK_HEAD_DIM - 1)) : 0;
  const int c1 = j0 < hd.kept ? (p.kept_idx[h * LEANK_HEAD_DIM + j0 + 1] & (LEANK_HEAD_DIM - 1)) : 0;
  const uint32_t kc = compact_k_word(kw, c0, c1);
  if (p.paged) {
    const int64_t page = p.block_table[static_cast<int64_t>(b) * p.pages_per_row + r / LEANK_PAGE_ROWS];
    uint16_t* base = p.pool + page * p.page_elems;
    const int64_t in = r % LEANK_PAGE_ROWS;
    if (j0 < hd.kept) reinterpret_cast<uint32_t*>(base + hd.k_off + in * hd.kept)[lane] = kc;
    store_v_row_word(base + hd.v_off, in, lane, vw);
    return;
  }
  const int64_t row = static_cast<int64_t>(b) * p.mid_cap + r;
  if (j0 < hd.kept) p.k_prun[(hd.k_off + row * hd.kept) / 2 + lane] = kc;
  store_v_row_word(p.v_mid + hd.v_off + static_cast<int64_t>(b) * p.v_mid_rows * LEANK_HEAD_DIM, r,
                   lane, vw);
}

__global__ __launch_bounds__(64 * kUnitsPerBlock) void pack_kernel(const PackParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kUnitsPerBlock + (threadIdx.x >> 6);
  if (unit >= p.n_units) return;  // whole wavefront leaves together
  const int64_t pair = unit / p.units_per_pair;
  const int64_t i = unit - pair * p.units_per_pair;
  const int b = static_cast<int>(pair / p.n_kv);
  const int h = static_cast<int>(pair - static_cast<int64_t>(b) * p.n_kv);
  uint32_t* ring_k = p.k_sl + (pair * p.slots) * kWordsPerRow;
  uint16_t* ring_v = p.v_sl + pair * p.v_sl_rows * LEANK_HEAD_DIM;

  int64_t t_old = p.t_old, t_new = p.t_new;
  if (p.row_pos) {
    t_old = p.row_pos[b];
    const int64_t cnt = p.row_count ? p.row_count[b] : p.n_new;
    // a row whose positions fall outside the cache is left untouched
    if (t_old < 0 || cnt < 0 || cnt > p.n_new || t_old + cnt > p.max_ctx) return;
    t_new = t_old + cnt;
  }

  if (p.mode == kMigrate) {
    const int64_t lo = max(static_cast<int64_t>(p.n_sink), t_old - p.window);
    const int64_t q = (p.row_pos ? lo : p.unit_lo) + i;
    if (q >= min(t_old, t_new - p.window)) return;  // this row moves fewer tokens
    const int64_t slot = p.n_sink + (q - p.n_sink) % p.window;
    const uint32_t kw = ring_k[slot * kWordsPerRow + lane];
    const uint32_t vw = load_v_row_word(ring_v, slot, lane);
    write_middle(p, b, h, q - p.n_sink, kw, vw, lane);
    return;
  }

  if (i >= t_new - t_old) return;  // this row appends fewer tokens
  const int64_t pos = t_old + i;
  const int64_t src = (pair * p.n_new + i) * kWordsPerRow + lane;
  const uint32_t kw = p.k_new[src];
  const uint32_t vw = p.v_new[src];
  if (pos < p.n_sink) {
    ring_k[pos * kWordsPerRow + lane] = kw;
    store_v_row_word(ring_v, pos, lane, vw);
    return;
  }
  if (p.mode == kPlace && pos < t_new - p.window) {
    if (!p.ring_only) write_middle(p, b, h, pos - p.n_sink, kw, vw, lane);  // already outside the window
    return;
  }
  const int64_t slot = p.n_sink + (pos - p.n_sink) % p.window;
  if (p.mode == kFused) {
    const int64_t leaving = pos - p.window;  // token held by this ring row until now
    if (leaving >= p.n_sink) {
      const uint32_t old_k = ring_k[slot * kWordsPerRow + lane];
      const uint32_t old_v = load_v_row_word(ring_v, slot, lane);
      write_middle(p, b, h, leaving - p.n_sink, old_k, old_v, lane);
    }
  }
  ring_k[slot * kWordsPerRow + lane] = kw;
  store_v_row_word(ring_v, slot, lane, vw);
}

int launch(PackParams& p, int64_t units_per_pair, int64_t pairs, hipStream_t s) {
  p.units_per_pair = units_per_pair;
  p.n_units = units_per_pair * pairs;
  const int64_t blocks = (p.n_units + kUnitsPerBlock - 1) / kUnitsPerBlock;
  if (blocks > INT32_MAX) return LEANK_EUNSUPPORTED;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(64 * kUnitsPerBlock),
                     0, s, p);
  LEANK_HIP_TRY(hipGetLastError());
  return LEANK_OK;
}

}  // namespace
}  // namespace leank

using namespace leank;

namespace {

int fill_params(const leank_layer_cache* c, const void* k_new, const void* v_new, int64_t n_new,
                PackParams* p) {
  memset(p, 0, sizeof(*p));
  p->k_new = static_cast<const uint32_t*>(k_new);
  p->v_new = static_cast<const uint32_t*>(v_new);
  p->k_sl = static_cast<uint32_t*>(c->k_sl);
  p->v_sl = static_cast<uint16_t*>(c->v_sl);
  p->k_prun = static_cast<uint32_t*>(c->k_prun);
  p->v_mid = static_cast<uint16_t*>(c->v_mid);
  p->kept_idx = c->kept_idx;
  p->n_new = n_new;
  p->mid_cap = c->mid_capacity;
  p->v_mid_rows = v_rows(c->mid_capacity);
  p->v_sl_rows = v_rows(static_cast<int64_t>(c->n_sink) + c->window);
  p->max_ctx = c->max_ctx;
  p->n_kv = c->n_kv_heads;
  p->n_sink = c->n_sink;
  p->window = c->window;
  p->slots = c->n_sink + c->window;
  p->paged = c->page_rows != 0;
  p->pool = static_cast<uint16_t*>(c->pool);
  p->block_table = c->block_table;
  p->page_elems = static_cast<int64_t>(c->page_bytes / 2);
  p->pages_per_row = c->pages_per_row;
  for (int h = 0; h < c->n_kv_heads; ++h) {
    p->heads[h].k_off = c->k_prun_off[h];
    p->heads[h].v_off = c->v_mid_off[h];
    p->heads[h].kept = c->kept_count[h];
  }
  return LEANK_OK;
}

}  // namespace

extern "C" int leank_pack_k(const leank_layer_cache* c, const void* k_new, const void* v_new,
                            int64_t pos0, int64_t n_new, void* stream) {
  int st = validate_cache(c, true);
  if (st != LEANK_OK) return st;
  if (pos0 < 0 || n_new < 0) return LEANK_EINVAL;
  if (n_new == 0) return LEANK_OK;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return LEANK_EINVAL;
  if (pos0 + n_new > c->max_ctx) return LEANK_ECAPACITY;

  PackParams p;
  fill_params(c, k_new, v_new, n_new, &p);
  p.t_old = pos0;
  p.t_new = pos0 + n_new;
  const int64_t pairs = static_cast<int64_t>(c->batch) * c->n_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (c->quant_bits != 0) {
    // low-bit middle: a prefill into an empty cache in bulk; any other
    // append token by token (each may complete a K group)
    if (pos0 != 0 || n_new == 1)
      return quant_append(c, k_new, v_new, pos0, n_new, nullptr, nullptr, c->max_ctx, s);
    p.ring_only = 1;
    p.mode = n_new <= c->window ? kFused : kPlace;
    st = launch(p, n_new, pairs, s);  // sink and window rows
    if (st != LEANK_OK) return st;
    return quant_pack_bulk(c, k_new, v_new, n_new, s);
  }

  if (c->window > 0 && n_new <= c->window) {
    p.mode = kFused;
    return launch(p, n_new, pairs, s);
  }
  if (c->window > 0) {
    // window tokens pushed out by this append move to the middle first
    const int64_t lo = std::max<int64_t>(c->n_sink, pos0 - c->window);
    const int64_t hi = std::min<int64_t>(pos0, pos0 + n_new - c->window);
    if (hi > lo) {
      p.mode = kMigrate;
      p.unit_lo = lo;
      st = launch(p, hi - lo, pairs, s);
      if (st != LEANK_OK) return st;
    }
  }
  p.mode = kPlace;
  p.unit_lo = 0;
  return launch(p, n_new, pairs, s);
}

extern "C" int leank_pack_k_rows(const leank_layer_cache* c, const void* k_new, const void* v_new,
                                 const int64_t* row_pos, const int32_t* row_count, int64_t n_new,
                                 void* stream) {
  int st = validate_cache(c, true);
  if (st != LEANK_OK) return st;
  if (n_new < 0 || !row_pos) return LEANK_EINVAL;
  if (n_new == 0) return LEANK_OK;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return LEANK_EINVAL;
  if (n_new > c->max_ctx) return LEANK_ECAPACITY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->quant_bits != 0)  // token by token per row
    return quant_append(c, k_new, v_new, 0, n_new, row_pos, row_count, c->max_ctx, s);

  PackParams p;
  fill_params(c, k_new, v_new, n_new, &p);
  p.row_pos = row_pos;
  p.row_count = row_count;
  const int64_t pairs = static_cast<int64_t>(c->batch) * c->n_kv_heads;
  if (c->window > 0 && n_new <= c->window) {
    p.mode = kFused;
    return launch(p, n_new, pairs, s);
  }
  if (c->window > 0) {
    p.mode = kMigrate;
    st = launch(p, std::min<int64_t>(c->window, n_new), pairs, s);
    if (st != LEANK_OK) return st;
  }
  p.mode = kPlace;
  return launch(p, n_new, pairs, s);
}
