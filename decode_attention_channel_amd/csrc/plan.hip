// Host-side entry points: status strings, layer plan (head grouping and
// cache layout, LeanK page section 3.1 items 1-2), work decomposition of a
// decode call, workspace sizing and algorithmic byte accounting.

#include <string.h>

#include <algorithm>

#include "common.h"

namespace leank {

namespace {

// Work-item sizing (compile-time tuning knobs; defaults measured on MI355X).
// Items are sized so that one decode call makes about kTargetCUs *
// LEANK_ITEMS_PER_CU of them, within [LEANK_ITEM_KB_MIN, LEANK_ITEM_KB_MAX].
// A call too small for that makes one round of the workgroups the chip runs
// at once (kTargetCUs * kRoundPerCU) instead, with items no smaller than the
// minimum: just over one round would leave a short second round running on
// a nearly idle chip.
#ifndef LEANK_ITEMS_PER_CU
#define LEANK_ITEMS_PER_CU 5
#endif
#ifndef LEANK_ITEM_KB_MIN
#define LEANK_ITEM_KB_MIN 128
#endif
#ifndef LEANK_ITEM_KB_MAX
#define LEANK_ITEM_KB_MAX 448
#endif

// Item sizing weighs the bytes of a low-bit middle row by
// LEANK_Q4_ROW_COST / LEANK_Q8_ROW_COST percent: a 4-bit row costs more
// time per byte than a bf16 row (its codes are expanded on the way into the
// matrix instructions).  Measured on the Llama batch-64 4K step with a
// 4-bit middle: 100 / 150 / 200 / 300 percent gave 76.5 / 76.4 / 72.6 /
// 77.5 us (at 200 the full-width rows of a pair make one item, not two);
// with an 8-bit middle 100 / 150 / 200 / 300 gave 89.5 / 91.4 / 91.6 /
// 95.5 us.
#ifndef LEANK_Q4_ROW_COST
#define LEANK_Q4_ROW_COST 200
#endif
#ifndef LEANK_Q8_ROW_COST
#define LEANK_Q8_ROW_COST 100
#endif

#ifndef LEANK_ONE_ROUND
#define LEANK_ONE_ROUND 1
#endif
#ifndef LEANK_BALANCE_ROUND
#define LEANK_BALANCE_ROUND 1
#endif
#ifndef LEANK_TAIL_PCT
#define LEANK_TAIL_PCT 15
#endif
#ifndef LEANK_TAIL_DIV
#define LEANK_TAIL_DIV 2
#endif
#ifndef LEANK_TAIL_MAX_KEPT
#define LEANK_TAIL_MAX_KEPT 64
#endif
#ifndef LEANK_SL_FIRST
#define LEANK_SL_FIRST 1
#endif

constexpr int64_t kTargetCUs = 256;  // compute units of an MI355X
constexpr int64_t kRoundPerCU = 3;   // split-kernel workgroups resident per compute unit
constexpr int64_t kRowQuantum = 64;  // item row counts are multiples of this
constexpr int64_t kItemBytesMin = int64_t{LEANK_ITEM_KB_MIN} << 10;
constexpr int64_t kItemBytesMax = int64_t{LEANK_ITEM_KB_MAX} << 10;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Rows per item for a stream whose rows take row_bytes: about `target`
// bytes per item, a multiple of kRowQuantum, at least kRowQuantum.
int64_t row_target(int64_t row_bytes, int64_t target) {
  int64_t rows = (target / row_bytes) / kRowQuantum * kRowQuantum;
  return std::max(rows, kRowQuantum);
}

// Splits `rows` rows into items of at most `target_rows` rows each (a
// multiple of kRowQuantum).  `bound` receives an item count that never
// decreases as `rows` grows (used for workspace sizing).
void split_rows(int64_t rows, int64_t target_rows, int32_t* n_items, int32_t* rows_per_item,
                int64_t* bound) {
  if (rows <= 0) {
    *n_items = 0;
    *rows_per_item = 0;
    *bound = 0;
    return;
  }
  int64_t n = ceil_div(rows, target_rows);
  int64_t per = ceil_div(ceil_div(rows, n), kRowQuantum) * kRowQuantum;
  *bound = n;
  *n_items = static_cast<int32_t>(ceil_div(rows, per));
  *rows_per_item = static_cast<int32_t>(per);
}

}  // namespace

int64_t middle_row_bytes(const leank_layer_cache* c, int kept) {
  if (c->quant_bits == 0) return 2 * static_cast<int64_t>(kept) + 2 * LEANK_HEAD_DIM;
  // codes of K and V, the row's V scale and minimum (K parameters are per group)
  return (static_cast<int64_t>(kept) + LEANK_HEAD_DIM) * c->quant_bits / 8 + 8;
}

namespace {
// Sizing weight of one middle row: its bytes, scaled for low-bit rows.
int64_t middle_row_cost(const leank_layer_cache* c, int kept) {
  const int64_t bytes = middle_row_bytes(c, kept);
  if (c->quant_bits == 4) return bytes * LEANK_Q4_ROW_COST / 100;
  if (c->quant_bits == 8) return bytes * LEANK_Q8_ROW_COST / 100;
  return bytes;
}
// Items a call over t_sl full-width and t_mid middle rows per pair makes
// when its items aim at `target` bytes (the split make_work_plan applies).
int64_t items_for_target(const leank_layer_cache* c, int32_t t_sl, int32_t t_mid, int step,
                         int64_t target) {
  int32_t n, rows;
  int64_t bound;
  split_rows(t_sl, row_target(4 * LEANK_HEAD_DIM, target), &n, &rows, &bound);
  if (step && n == 0) n = 1;
  int64_t per_b = static_cast<int64_t>(n) * c->n_kv_heads;
  for (int h = 0; h < c->n_kv_heads; ++h) {
    const int kept = c->kept_count[h];
    if (kept <= 0) continue;
    int64_t r = row_target(middle_row_cost(c, kept), target);
    if (c->page_rows) r = std::min<int64_t>(r, 64 * LEANK_PAGE_ROWS);
    split_rows(t_mid, r, &n, &rows, &bound);
    per_b += n;
  }
  return per_b * c->batch;
}

// Balanced one round: `n_items` items (a multiple of the compute units)
// over the segments of one batch row -- the full-width rows of each of the
// n_kv heads (one shared item count) and the middle of each live head --
// with nearly equal bytes per item.  Each segment takes its share of the
// items by largest remainder, at most `cap` items and at least one; the
// result is written to the plan fields.  Returns false (plan untouched)
// when the row's items cannot be placed.
bool balance_round(const leank_layer_cache* c, int32_t t_sl, int32_t t_mid, int step,
                   int64_t per_b, const int32_t* cap_mid, int32_t cap_sl, WorkPlan* w) {
  const int H = c->n_kv_heads;
  const double fw_bytes = static_cast<double>(t_sl) * 4 * LEANK_HEAD_DIM;
  double mid_bytes[LEANK_MAX_KV_HEADS] = {0};
  double total = fw_bytes * H;
  for (int h = 0; h < H; ++h)
    if (c->kept_count[h] > 0) {
      mid_bytes[h] = static_cast<double>(t_mid) * middle_row_cost(c, c->kept_count[h]);
      total += mid_bytes[h];
    }
  if (total <= 0) return false;
  const double per_item = total / static_cast<double>(per_b);
  const int32_t sl_min = (t_sl > 0 || step) ? 1 : 0;
  int32_t n_sl = t_sl > 0 ? static_cast<int32_t>(std::llround(fw_bytes / per_item)) : 0;
  n_sl = std::min(std::max(n_sl, sl_min), std::max(cap_sl, sl_min));
  int32_t n_mid[LEANK_MAX_KV_HEADS] = {0};
  int64_t sum = static_cast<int64_t>(H) * n_sl;
  for (int h = 0; h < H; ++h)
    if (mid_bytes[h] > 0 && t_mid > 0) {
      n_mid[h] = std::min(std::max<int32_t>(1, static_cast<int32_t>(std::llround(mid_bytes[h] / per_item))),
                          std::max(cap_mid[h], 1));
      sum += n_mid[h];
    }
  // largest remainder: take items from the segment with the smallest items,
  // give them to the one with the largest, until the row holds per_b
  for (int it = 0; it < 4 * LEANK_MAX_KV_HEADS * 64 && sum != per_b; ++it) {
    int best = -2;  // -1: the full-width segments, h: head h's middle
    double best_size = sum > per_b ? 1e300 : -1.0;
    if (n_sl > 0) {
      const double size = fw_bytes / n_sl;
      const bool ok = sum > per_b ? (n_sl > sl_min && sum - H >= per_b - H) : (n_sl < cap_sl && sum + H <= per_b);
      if (ok && (sum > per_b ? size < best_size : size > best_size)) best = -1, best_size = size;
    }
    for (int h = 0; h < H; ++h) {
      if (n_mid[h] == 0) continue;
      const double size = mid_bytes[h] / n_mid[h];
      const bool ok = sum > per_b ? n_mid[h] > 1 : n_mid[h] < cap_mid[h];
      if (ok && (sum > per_b ? size < best_size : size > best_size)) best = h, best_size = size;
    }
    if (best == -2) break;
    const int d = sum > per_b ? -1 : 1;
    if (best == -1) {
      n_sl += d;
      sum += d * H;
    } else {
      n_mid[best] += d;
      sum += d;
    }
  }
  if (sum > per_b) return false;
  auto rows_for = [](int32_t rows, int32_t n, int32_t* n_out, int32_t* rows_out) {
    if (rows <= 0 || n <= 0) {
      *n_out = n > 0 ? n : 0;
      *rows_out = 0;
      return;
    }
    const int64_t per = ceil_div(ceil_div(rows, n), kRowQuantum) * kRowQuantum;
    *rows_out = static_cast<int32_t>(per);
    *n_out = static_cast<int32_t>(ceil_div(rows, per));
  };
  rows_for(t_sl, n_sl, &w->n_sl_items, &w->sl_rows);
  if (step && w->n_sl_items == 0) w->n_sl_items = 1;
  for (int h = 0; h < H; ++h) rows_for(t_mid, n_mid[h], &w->n_mid[h], &w->mid_rows[h]);
  return true;
}

}  // namespace

int validate_cache(const leank_layer_cache* c, bool need_buffers) {
  if (!c) return LEANK_EINVAL;
  if (c->head_dim != LEANK_HEAD_DIM) return LEANK_EUNSUPPORTED;
  if (c->n_kv_heads < 1 || c->n_kv_heads > LEANK_MAX_KV_HEADS) return LEANK_EINVAL;
  if (c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads) return LEANK_EINVAL;
  if (c->n_q_heads / c->n_kv_heads > LEANK_MAX_GROUP) return LEANK_EUNSUPPORTED;
  if (c->batch < 1 || c->n_sink < 0 || c->window < 0) return LEANK_EINVAL;
  if (static_cast<int64_t>(c->n_sink) + c->window < 1) return LEANK_EINVAL;
  if (c->max_ctx < 1 || c->max_ctx > INT32_MAX) return LEANK_EINVAL;
  if (c->mid_capacity != std::max<int64_t>(0, c->max_ctx - c->n_sink - c->window)) return LEANK_EINVAL;
  const bool quant = c->quant_bits != 0;
  if (quant && c->quant_bits != 4 && c->quant_bits != 8) return LEANK_EINVAL;
  if (quant && c->quant_group != LEANK_QUANT_GROUP) return LEANK_EINVAL;
  const bool paged = c->page_rows != 0;
  if (paged) {
    // canonical page layouts: bf16, K of the live heads in group order, then
    // their V blocks; low-bit, as QPageLayout describes (staging not paged)
    if (c->page_rows != LEANK_PAGE_ROWS || c->n_pages < 1) return LEANK_EINVAL;
    if (c->pages_per_row != (c->mid_capacity + LEANK_PAGE_ROWS - 1) / LEANK_PAGE_ROWS) return LEANK_EINVAL;
    int64_t kept_sum = 0, n_live = 0;
    for (int h = 0; h < c->n_kv_heads; ++h)
      if (c->kept_count[h] > 0) kept_sum += c->kept_count[h], ++n_live;
    const QPageLayout ql = q_page_layout(kept_sum, n_live, quant ? c->quant_bits : 8);
    int64_t k_pre = 0, rank = 0;
    for (int i = 0; i < c->n_kv_heads; ++i) {
      const int h = c->group_order[i];
      if (h < 0 || h >= c->n_kv_heads) return LEANK_EINVAL;
      if (c->kept_count[h] <= 0) continue;
      if (!quant) {
        if (c->k_prun_off[h] != LEANK_PAGE_ROWS * k_pre ||
            c->v_mid_off[h] != LEANK_PAGE_ROWS * (kept_sum + rank * LEANK_HEAD_DIM))
          return LEANK_EINVAL;
      } else if (c->k_q_off[h] != LEANK_PAGE_ROWS * k_pre * c->quant_bits / 8 ||
                 c->k_qp_off[h] != (ql.kc_bytes + 8 * k_pre) / 4 ||
                 c->v_q_off[h] != ql.kc_bytes + ql.kp_bytes + rank * ql.vc_head ||
                 c->v_qp_off[h] != (ql.kc_bytes + ql.kp_bytes + n_live * ql.vc_head + rank * ql.vp_head) / 4 ||
                 c->k_stage_off[h] != static_cast<int64_t>(c->batch) * LEANK_QUANT_GROUP * k_pre) {
        return LEANK_EINVAL;
      }
      k_pre += c->kept_count[h];
      ++rank;
    }
    const int64_t page_bytes =
        quant ? ql.page_bytes : LEANK_PAGE_ROWS * (2 * kept_sum + 2 * LEANK_HEAD_DIM * n_live);
    if (static_cast<int64_t>(c->page_bytes) != page_bytes ||
        c->pool_bytes != c->page_bytes * static_cast<uint64_t>(c->n_pages))
      return LEANK_EINVAL;
  }
  int live = 0;
  for (int h = 0; h < c->n_kv_heads; ++h) {
    int k = c->kept_count[h];
    if (k < 0 || k > LEANK_HEAD_DIM) return LEANK_EINVAL;
    if (k % LEANK_CHANNEL_QUANTUM) return LEANK_EUNSUPPORTED;
    if (k > 0) {
      ++live;
      if (!quant) {
        if (c->k_prun_off[h] < 0 || c->v_mid_off[h] < 0) return LEANK_EINVAL;
        // (paged caches: offsets within a page, checked against the canonical layout above)
        if (!paged && (c->k_prun_off[h] % LEANK_CHANNEL_QUANTUM ||
                       c->v_mid_off[h] % (LEANK_HEAD_DIM * LEANK_V_BLOCK)))
          return LEANK_EINVAL;
      } else {
        if (c->k_q_off[h] < 0 || c->k_qp_off[h] < 0 || c->k_stage_off[h] < 0 ||
            c->v_q_off[h] < 0 || c->v_qp_off[h] < 0)
          return LEANK_EINVAL;
        // 16-byte aligned code and parameter segments, 8-byte aligned row parameters
        if (c->k_q_off[h] % 16 || c->k_qp_off[h] % 4 || c->k_stage_off[h] % 8 ||
            c->v_q_off[h] % 16 || c->v_qp_off[h] % 2)
          return LEANK_EINVAL;
      }
    }
  }
  if (live != c->n_live) return LEANK_EINVAL;
  if (need_buffers) {
    if (!c->k_sl || !c->v_sl || !c->kept_idx) return LEANK_EINVAL;
    if (!aligned16(c->k_sl) || !aligned16(c->v_sl)) return LEANK_EINVAL;
    if (paged) {
      if (c->pool_bytes && (!c->pool || !aligned16(c->pool))) return LEANK_EINVAL;
      if (c->pages_per_row > 0 && !c->block_table) return LEANK_EINVAL;
      if (quant && c->k_stage_bytes && (!c->k_stage || !aligned16(c->k_stage))) return LEANK_EINVAL;
    } else if (!quant) {
      if (c->k_prun_bytes && (!c->k_prun || !aligned16(c->k_prun))) return LEANK_EINVAL;
      if (c->v_mid_bytes && (!c->v_mid || !aligned16(c->v_mid))) return LEANK_EINVAL;
    } else {
      const void* bufs[5] = {c->k_q, c->k_qp, c->k_stage, c->v_q, c->v_qp};
      const uint64_t sizes[5] = {c->k_q_bytes, c->k_qp_bytes, c->k_stage_bytes, c->v_q_bytes,
                                 c->v_qp_bytes};
      for (int i = 0; i < 5; ++i)
        if (sizes[i] && (!bufs[i] || !aligned16(bufs[i]))) return LEANK_EINVAL;
    }
  }
  return LEANK_OK;
}

int make_work_plan(const leank_layer_cache* c, int64_t ctx_len, int step, WorkPlan* w) {
  memset(w, 0, sizeof(*w));
  w->step = step;
  const int64_t slots = static_cast<int64_t>(c->n_sink) + c->window;
  w->group = c->n_q_heads / c->n_kv_heads;
  w->t_sl = static_cast<int32_t>(std::min<int64_t>(ctx_len, slots));
  w->t_mid = static_cast<int32_t>(std::max<int64_t>(0, ctx_len - slots));
  // bytes the call streams (K and V rows of both regions; low-bit middle
  // rows weighted by their cost)
  int64_t stream_bytes = static_cast<int64_t>(c->batch) * c->n_kv_heads * w->t_sl * 4 * LEANK_HEAD_DIM;
  for (int h = 0; h < c->n_kv_heads; ++h)
    if (c->kept_count[h] > 0)
      stream_bytes += static_cast<int64_t>(c->batch) * w->t_mid * middle_row_cost(c, c->kept_count[h]);
  int64_t target = stream_bytes / (kTargetCUs * LEANK_ITEMS_PER_CU);
  if (target < kItemBytesMin) target = std::max(kItemBytesMin, stream_bytes / (kTargetCUs * kRoundPerCU));
  target = std::min(kItemBytesMax, target);
  // One round: the resident workgroups (kTargetCUs * kRoundPerCU) take the
  // items in rounds, and a second round that is not full runs with part of
  // the chip idle.  A bf16 call whose items fill more than one round but
  // less than two is planned as one round of larger items instead.
  // Measured (MI355X): the 32-layer 128K-token batch-1 token 1061 -> 987
  // us, the Qwen2.5-7B-shaped batch-16 32K step 95.2 -> 93.0 us.  Calls of
  // two rounds or more, and low-bit middles, keep their items: folding them
  // into whole rounds measured slower (Llama batch-64 4K at 0% pruning
  // 189.6 -> 198.9 us, its 8-bit middle 88.7 -> 99.0 us).
  if (LEANK_ONE_ROUND && c->quant_bits == 0) {
    const int64_t round = kTargetCUs * kRoundPerCU;
    int64_t items = items_for_target(c, w->t_sl, w->t_mid, step, target);
    if (items > round && items < 2 * round) {
      for (int it = 0; it < 64 && items > round; ++it) {
        target += target / 8 + 1;
        items = items_for_target(c, w->t_sl, w->t_mid, step, target);
      }
    }
  }

  // item counts at the smallest item size bound the workspace for any ctx <= this one
  int64_t bound_per_b = 0, b, unused_n, unused_rows;
  int32_t n32, rows32;
  split_rows(w->t_sl, row_target(4 * LEANK_HEAD_DIM, kItemBytesMin), &n32, &rows32, &b);
  bound_per_b += b * c->n_kv_heads;
  split_rows(w->t_sl, row_target(4 * LEANK_HEAD_DIM, target), &w->n_sl_items, &w->sl_rows, &unused_n);
  if (step && w->n_sl_items == 0) {  // item 0 carries the append even over no cached rows
    w->n_sl_items = 1;
    bound_per_b += c->n_kv_heads;
  }
  const int32_t cap_sl = static_cast<int32_t>(b);  // full-width items at the smallest size
  int32_t cap_mid[LEANK_MAX_KV_HEADS] = {0};
  int64_t items = static_cast<int64_t>(w->n_sl_items) * c->n_kv_heads;
  for (int h = 0; h < c->n_kv_heads; ++h) {
    const int kept = c->kept_count[h];
    if (kept > 0) {
      const int64_t row_bytes = middle_row_cost(c, kept);
      split_rows(w->t_mid, row_target(row_bytes, kItemBytesMin), &n32, &rows32, &b);
      bound_per_b += b;
      cap_mid[h] = static_cast<int32_t>(b);
      int64_t rows = row_target(row_bytes, target);
      // a paged item reads its page list from LDS: at most 64 pages
      if (c->page_rows) rows = std::min<int64_t>(rows, 64 * LEANK_PAGE_ROWS);
      split_rows(w->t_mid, rows, &w->n_mid[h], &w->mid_rows[h], &unused_n);
      items += w->n_mid[h];
    }
  }
  items *= c->batch;
  // Balanced round: the compute units share HBM bandwidth per unit, so a
  // unit running three workgroups of a round serves each more slowly than
  // one running two, and a round ends when its most loaded unit does.  A
  // bf16 call of one round with at least 2 * kItemBytesMin bytes per unit
  // makes exactly 2 or 3 items per unit (as many as keep items at or above
  // kItemBytesMin), of nearly equal bytes.  Measured (MI355X): the
  // Qwen2.5-7B-shaped batch-16 32K step 93.0 -> 89.9 us (688 -> 768 items);
  // one item per unit was slower (the 128K-token layer with one live head:
  // 20.9 -> 23.1 us with 256 items instead of 475).  Paged middles keep the
  // plan above (an item's pages are capped).
  const int64_t units_items = stream_bytes / (kTargetCUs * kItemBytesMin);
  if (LEANK_BALANCE_ROUND && c->quant_bits == 0 && !c->page_rows &&
      items <= kTargetCUs * kRoundPerCU && units_items >= 2) {
    const int64_t per_b = kTargetCUs * std::min<int64_t>(kRoundPerCU, units_items) / c->batch;
    if (per_b >= 1) balance_round(c, w->t_sl, w->t_mid, step, per_b, cap_mid, cap_sl, w);
  }
  for (int h = 0; h < c->n_kv_heads; ++h) {
    w->n_mid_b[h] = w->n_mid[h];
    w->mid_rows_t[h] = w->mid_rows[h];
  }
  // Tail items: a launch of more than one round of items ends in a drain,
  // the slots emptying one by one as their last items finish at different
  // times.  So the last LEANK_TAIL_PCT percent of each middle segment is cut
  // into items LEANK_TAIL_DIV times smaller than its (resized) bulk items,
  // and every batch row's tail items are dispatched after all bulk items:
  // the slots that free up first take the smaller pieces.  Records keep
  // their order within each (batch row, head), so the merge order does not
  // change.  A segment keeps its items when its tail would not fit the item
  // count the workspace is sized for.  Measured (MI355X, against no tail):
  // the Llama batch-64 4K step 113.7 -> 110.9 us, its paged middle 118.1 ->
  // 114.6 us, its 8-bit middle 90.0 -> 88.5 us, 4-bit unchanged; heads
  // keeping more than LEANK_TAIL_MAX_KEPT channels keep their items (at 0%
  // pruning the same rule measured 190.4 -> 199.6 us).
  if (LEANK_TAIL_PCT > 0 && items > kTargetCUs * kRoundPerCU) {
    for (int h = 0; h < c->n_kv_heads; ++h) {
      const int64_t rows = w->t_mid;
      if (c->kept_count[h] <= 0 || c->kept_count[h] > LEANK_TAIL_MAX_KEPT || w->n_mid[h] < 2) continue;
      // bulk items resized so that they cover about 100 - LEANK_TAIL_PCT
      // percent of the rows
      const int64_t bulk_rows = rows * (100 - LEANK_TAIL_PCT) / 100;
      const int64_t n_b = std::max<int64_t>(1, (bulk_rows + w->mid_rows[h] / 2) / w->mid_rows[h]);
      const int64_t R = ceil_div(ceil_div(bulk_rows, n_b), kRowQuantum) * kRowQuantum;
      if (n_b * R >= rows || (c->page_rows && R > 64 * LEANK_PAGE_ROWS)) continue;
      const int64_t r_t = std::max(kRowQuantum, R / LEANK_TAIL_DIV / kRowQuantum * kRowQuantum);
      const int64_t n_t = ceil_div(rows - n_b * R, r_t);
      if (n_b + n_t > cap_mid[h]) continue;
      w->mid_rows[h] = static_cast<int32_t>(R);
      w->n_mid_b[h] = static_cast<int32_t>(n_b);
      w->mid_rows_t[h] = static_cast<int32_t>(r_t);
      w->n_mid[h] = static_cast<int32_t>(n_b + n_t);
    }
  }
  // Longest items first: a launch of more than one round dispatches its
  // full-width items (every batch row's) ahead of the middle ones when a
  // full-width item costs more than any bulk middle item, so that the long
  // items do not start late and end the launch after the short ones.
  // Measured (MI355X): the Llama batch-64 4K step with a 4-bit middle
  // (full-width items 288 KB of bf16 rows, bulk middle items 1536 rows of
  // 4-bit codes) 72.7 -> 70.5 us, with an 8-bit middle 88.4 -> 87.0 us;
  // bf16 middles keep the interleaved order (their bulk items are larger).
  w->sl_first = 0;
  if (LEANK_SL_FIRST && w->n_sl_items > 0 && items > kTargetCUs * kRoundPerCU) {
    const int64_t sl_cost = static_cast<int64_t>(w->sl_rows) * 4 * LEANK_HEAD_DIM;
    int64_t mid_cost = 0;
    for (int h = 0; h < c->n_kv_heads; ++h)
      if (c->kept_count[h] > 0 && w->n_mid_b[h] > 0)
        mid_cost = std::max(mid_cost, static_cast<int64_t>(w->mid_rows[h]) * middle_row_cost(c, c->kept_count[h]));
    w->sl_first = sl_cost > mid_cost ? 1 : 0;
  }
  int32_t base = 0;
  w->bulk_per_b = 0;
  w->tail_per_b = 0;
  for (int h = 0; h < c->n_kv_heads; ++h) {
    w->head_base[h] = base;
    base += w->n_sl_items + w->n_mid[h];
    w->bulk_per_b += w->n_sl_items + w->n_mid_b[h];
    w->tail_per_b += w->n_mid[h] - w->n_mid_b[h];
  }
  (void)unused_rows;
  w->head_base[c->n_kv_heads] = base;
  w->items_per_b = base;
  w->n_items = static_cast<int64_t>(base) * c->batch;

  w->partial_stride = w->group * LEANK_HEAD_DIM + ((2 * w->group + 3) / 4) * 4;
  const int64_t bound_items = bound_per_b * c->batch;
  w->partial_bytes = static_cast<size_t>(bound_items) * w->partial_stride * sizeof(float);
  w->workspace_bytes = std::max<size_t>(256, (w->partial_bytes + 255) / 256 * 256);
  return LEANK_OK;
}

}  // namespace leank

using namespace leank;

extern "C" const char* leank_status_string(int status) {
  switch (status) {
    case LEANK_OK: return "LEANK_OK";
    case LEANK_EINVAL: return "LEANK_EINVAL: invalid argument";
    case LEANK_EUNSUPPORTED: return "LEANK_EUNSUPPORTED: shape outside what the kernels implement";
    case LEANK_ECAPACITY: return "LEANK_ECAPACITY: position beyond the cache capacity";
    case LEANK_EWORKSPACE: return "LEANK_EWORKSPACE: workspace missing or too small";
    case LEANK_EHIP: return "LEANK_EHIP: HIP runtime or launch failure";
    default: return "unknown leank status";
  }
}

extern "C" int leank_abi_version(void) { return LEANK_ABI_VERSION; }

extern "C" size_t leank_layer_cache_size(void) { return sizeof(leank_layer_cache); }

extern "C" int leank_plan_layer(const int32_t* kept_count_host, int32_t batch, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, int32_t n_sink,
                                int32_t window, int64_t max_ctx, leank_layer_cache* out) {
  if (!kept_count_host || !out) return LEANK_EINVAL;
  leank_layer_cache c;
  memset(&c, 0, sizeof(c));
  c.batch = batch;
  c.n_q_heads = n_q_heads;
  c.n_kv_heads = n_kv_heads;
  c.head_dim = head_dim;
  c.n_sink = n_sink;
  c.window = window;
  c.max_ctx = max_ctx;
  if (n_kv_heads < 1 || n_kv_heads > LEANK_MAX_KV_HEADS) return LEANK_EINVAL;
  c.mid_capacity = std::max<int64_t>(0, max_ctx - static_cast<int64_t>(n_sink) - window);

  int order[LEANK_MAX_KV_HEADS];
  for (int h = 0; h < n_kv_heads; ++h) {
    c.kept_count[h] = kept_count_host[h];
    order[h] = h;
    c.k_prun_off[h] = -1;
    c.v_mid_off[h] = -1;
  }
  // Head grouping: live heads by kept count (descending, then id), dead heads last.
  std::stable_sort(order, order + n_kv_heads, [&](int a, int b) {
    return c.kept_count[a] > c.kept_count[b];
  });
  int64_t k_off = 0, v_off = 0;
  for (int n = 0; n < n_kv_heads; ++n) {
    const int h = order[n];
    c.group_order[n] = h;
    const int kept = c.kept_count[h];
    if (kept <= 0) continue;
    ++c.n_live;
    c.k_prun_off[h] = k_off;
    c.v_mid_off[h] = v_off;
    k_off += static_cast<int64_t>(batch) * c.mid_capacity * kept;
    v_off += static_cast<int64_t>(batch) * v_rows(c.mid_capacity) * LEANK_HEAD_DIM;
  }
  const int64_t slots = static_cast<int64_t>(n_sink) + window;
  c.k_sl_bytes = static_cast<uint64_t>(batch) * n_kv_heads * slots * LEANK_HEAD_DIM * 2;
  c.v_sl_bytes = static_cast<uint64_t>(batch) * n_kv_heads * v_rows(slots) * LEANK_HEAD_DIM * 2;
  c.k_prun_bytes = static_cast<uint64_t>(k_off) * 2;
  c.v_mid_bytes = static_cast<uint64_t>(v_off) * 2;
  int st = validate_cache(&c, false);
  if (st != LEANK_OK) return st;
  *out = c;
  return LEANK_OK;
}

extern "C" int leank_plan_layer_q(const int32_t* kept_count_host, int32_t batch,
                                  int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                  int32_t n_sink, int32_t window, int64_t max_ctx,
                                  int32_t quant_bits, leank_layer_cache* out) {
  if (quant_bits != 0 && quant_bits != 4 && quant_bits != 8) return LEANK_EUNSUPPORTED;
  if (!out) return LEANK_EINVAL;
  leank_layer_cache c;
  int st = leank_plan_layer(kept_count_host, batch, n_q_heads, n_kv_heads, head_dim, n_sink,
                            window, max_ctx, &c);
  if (st != LEANK_OK || quant_bits == 0) {
    if (st == LEANK_OK) *out = c;
    return st;
  }
  c.quant_bits = quant_bits;
  c.quant_group = LEANK_QUANT_GROUP;
  const int64_t groups = (c.mid_capacity + LEANK_QUANT_GROUP - 1) / LEANK_QUANT_GROUP;
  const int64_t g_rows = groups * LEANK_QUANT_GROUP;
  int64_t kq = 0, kqp = 0, ks = 0, vq = 0, vqp = 0;
  for (int h = 0; h < n_kv_heads; ++h) {
    c.k_prun_off[h] = c.v_mid_off[h] = -1;
    c.k_q_off[h] = c.k_qp_off[h] = c.k_stage_off[h] = c.v_q_off[h] = c.v_qp_off[h] = -1;
  }
  for (int n = 0; n < n_kv_heads; ++n) {
    const int h = c.group_order[n];
    const int64_t kept = c.kept_count[h];
    if (kept <= 0) continue;
    c.k_q_off[h] = kq;
    c.k_qp_off[h] = kqp;
    c.k_stage_off[h] = ks;
    c.v_q_off[h] = vq;
    c.v_qp_off[h] = vqp;
    kq += static_cast<int64_t>(batch) * g_rows * kept * quant_bits / 8;
    kqp += static_cast<int64_t>(batch) * groups * kept * 2;
    ks += static_cast<int64_t>(batch) * LEANK_QUANT_GROUP * kept;
    vq += static_cast<int64_t>(batch) * v_rows(c.mid_capacity) * LEANK_HEAD_DIM * quant_bits / 8;
    vqp += static_cast<int64_t>(batch) * c.mid_capacity * 2;
  }
  c.k_prun_bytes = c.v_mid_bytes = 0;
  c.k_q_bytes = static_cast<uint64_t>(kq);
  c.k_qp_bytes = static_cast<uint64_t>(kqp) * 4;
  c.k_stage_bytes = static_cast<uint64_t>(ks) * 2;
  c.v_q_bytes = static_cast<uint64_t>(vq);
  c.v_qp_bytes = static_cast<uint64_t>(vqp) * 4;
  st = validate_cache(&c, false);
  if (st != LEANK_OK) return st;
  *out = c;
  return LEANK_OK;
}

extern "C" int leank_plan_layer_paged(const int32_t* kept_count_host, int32_t batch,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                      int32_t n_sink, int32_t window, int64_t max_ctx,
                                      int64_t n_pages, leank_layer_cache* out) {
  if (!out || n_pages < 1) return LEANK_EINVAL;
  leank_layer_cache c;
  int st = leank_plan_layer(kept_count_host, batch, n_q_heads, n_kv_heads, head_dim, n_sink,
                            window, max_ctx, &c);
  if (st != LEANK_OK) return st;
  int64_t kept_sum = 0;
  for (int h = 0; h < n_kv_heads; ++h) kept_sum += std::max(0, c.kept_count[h]);
  int64_t k_pre = 0, rank = 0;
  for (int h = 0; h < n_kv_heads; ++h) c.k_prun_off[h] = c.v_mid_off[h] = -1;
  for (int i = 0; i < n_kv_heads; ++i) {
    const int h = c.group_order[i];
    if (c.kept_count[h] <= 0) continue;
    c.k_prun_off[h] = LEANK_PAGE_ROWS * k_pre;
    c.v_mid_off[h] = LEANK_PAGE_ROWS * (kept_sum + rank * LEANK_HEAD_DIM);
    k_pre += c.kept_count[h];
    ++rank;
  }
  c.k_prun_bytes = c.v_mid_bytes = 0;
  c.page_rows = LEANK_PAGE_ROWS;
  c.pages_per_row = static_cast<int32_t>((c.mid_capacity + LEANK_PAGE_ROWS - 1) / LEANK_PAGE_ROWS);
  c.n_pages = n_pages;
  c.page_bytes = static_cast<uint64_t>(LEANK_PAGE_ROWS) * (2 * kept_sum + 2 * LEANK_HEAD_DIM * rank);
  c.pool_bytes = c.page_bytes * static_cast<uint64_t>(n_pages);
  st = validate_cache(&c, false);
  if (st != LEANK_OK) return st;
  *out = c;
  return LEANK_OK;
}

extern "C" int leank_plan_layer_paged_q(const int32_t* kept_count_host, int32_t batch,
                                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                        int32_t n_sink, int32_t window, int64_t max_ctx,
                                        int64_t n_pages, int32_t quant_bits,
                                        leank_layer_cache* out) {
  if (quant_bits == 0)
    return leank_plan_layer_paged(kept_count_host, batch, n_q_heads, n_kv_heads, head_dim, n_sink,
                                  window, max_ctx, n_pages, out);
  if (!out || n_pages < 1) return LEANK_EINVAL;
  leank_layer_cache c;
  int st = leank_plan_layer_q(kept_count_host, batch, n_q_heads, n_kv_heads, head_dim, n_sink,
                              window, max_ctx, quant_bits, &c);
  if (st != LEANK_OK) return st;
  int64_t kept_sum = 0, n_live = 0;
  for (int h = 0; h < n_kv_heads; ++h)
    if (c.kept_count[h] > 0) kept_sum += c.kept_count[h], ++n_live;
  const QPageLayout ql = q_page_layout(kept_sum, n_live, quant_bits);
  int64_t k_pre = 0, rank = 0;
  for (int i = 0; i < n_kv_heads; ++i) {
    const int h = c.group_order[i];
    if (c.kept_count[h] <= 0) continue;
    c.k_q_off[h] = LEANK_PAGE_ROWS * k_pre * quant_bits / 8;
    c.k_qp_off[h] = (ql.kc_bytes + 8 * k_pre) / 4;
    c.v_q_off[h] = ql.kc_bytes + ql.kp_bytes + rank * ql.vc_head;
    c.v_qp_off[h] = (ql.kc_bytes + ql.kp_bytes + n_live * ql.vc_head + rank * ql.vp_head) / 4;
    k_pre += c.kept_count[h];
    ++rank;
  }
  c.k_q_bytes = c.k_qp_bytes = c.v_q_bytes = c.v_qp_bytes = 0;  // the middle lives in pages
  c.page_rows = LEANK_PAGE_ROWS;
  c.pages_per_row = static_cast<int32_t>((c.mid_capacity + LEANK_PAGE_ROWS - 1) / LEANK_PAGE_ROWS);
  c.n_pages = n_pages;
  c.page_bytes = static_cast<uint64_t>(ql.page_bytes);
  c.pool_bytes = c.page_bytes * static_cast<uint64_t>(n_pages);
  st = validate_cache(&c, false);
  if (st != LEANK_OK) return st;
  *out = c;
  return LEANK_OK;
}


extern "C" int leank_workspace_bytes(const leank_layer_cache* cache, int64_t ctx_len,
                                     size_t* bytes_out) {
  int st = validate_cache(cache, false);
  if (st != LEANK_OK) return st;
  if (!bytes_out || ctx_len < 1) return LEANK_EINVAL;
  if (ctx_len > cache->max_ctx) return LEANK_ECAPACITY;
  WorkPlan w;
  make_work_plan(cache, ctx_len, 0, &w);
  *bytes_out = w.workspace_bytes;
  return LEANK_OK;
}

extern "C" int leank_decode_bytes(const leank_layer_cache* c, int64_t ctx_len, int64_t* bytes_out) {
  int st = validate_cache(c, false);
  if (st != LEANK_OK) return st;
  if (!bytes_out || ctx_len < 1) return LEANK_EINVAL;
  if (ctx_len > c->max_ctx) return LEANK_ECAPACITY;
  const int64_t slots = static_cast<int64_t>(c->n_sink) + c->window;
  const int64_t t_sl = std::min<int64_t>(ctx_len, slots);
  const int64_t t_mid = std::max<int64_t>(0, ctx_len - slots);
  const int64_t bq = static_cast<int64_t>(c->batch) * c->n_q_heads * LEANK_HEAD_DIM;
  int64_t kept_sum = 0;
  for (int h = 0; h < c->n_kv_heads; ++h) kept_sum += c->kept_count[h];
  int64_t bytes = bq * 2 + bq * 4;
  bytes += 2 * static_cast<int64_t>(c->batch) * c->n_kv_heads * t_sl * LEANK_HEAD_DIM * 2;
  if (c->quant_bits == 0) {
    bytes += static_cast<int64_t>(c->batch) * t_mid * kept_sum * 2;
    bytes += static_cast<int64_t>(c->batch) * c->n_live * t_mid * LEANK_HEAD_DIM * 2;
  } else {
    // complete K groups as codes + per-channel (scale, min); the open group bf16;
    // every middle V row as codes + its (scale, min)
    const int64_t q = c->quant_bits;
    const int64_t groups = t_mid / LEANK_QUANT_GROUP;
    const int64_t stage = t_mid - groups * LEANK_QUANT_GROUP;
    bytes += static_cast<int64_t>(c->batch) *
             (groups * LEANK_QUANT_GROUP * kept_sum * q / 8 + groups * kept_sum * 8 + stage * kept_sum * 2);
    bytes += static_cast<int64_t>(c->batch) * c->n_live * t_mid * (LEANK_HEAD_DIM * q / 8 + 8);
  }
  *bytes_out = bytes;
  return LEANK_OK;
}
