// The tokens a fused decode step appends and moves, and where the middle
// rows they land in live.
#pragma once

#include "decode_base.h"

namespace leank {

// The append of a fused decode step for one (batch row, KV head) pair
// (LeanK page, section 3.1 item 2): the token at position pos goes to its
// sink or ring row (with no window, to the middle), and the token it pushes
// out of the window, ring row `slot`, moves its kept K channels and -- for
// a live head -- its V to the middle.  The regular items of the call
// cover the rows cached before the append, minus that ring row; the two
// tokens are scored by the pair's full-width item 0, which stages them in
// LDS before its tile loop and writes the append after it.  V rows are
// written as whole 8-row blocks (read in the prologue, one row replaced in
// LDS, written back with 16-byte stores): a single row of a block is 128
// scattered 2-byte pieces, which the memory system handles far more slowly
// than the 2 KiB block.
struct StepTokens {
  bool ok;        // the row takes part (its position lies in the plan)
  bool new_full;  // the new token is a sink or window row (full width)
  bool new_in;    // the new token is attended (not a middle token of a dead head)
  bool leave_in;  // a token leaves the window of a live head
  bool to_ring;   // the new token is written to a sink or ring row
  int pos;
  int slot;       // ring row of the new token (and of the leaving one)
  int mid_row;    // middle row written by the append, -1 for none
};

__device__ __forceinline__ StepTokens step_tokens(const DecodeParams& p, int b, bool live) {
  StepTokens st;
  const int64_t pos = p.row_pos ? uniform64(p.row_pos[b]) : p.step_pos;
  st.ok = pos >= 0 && pos <= p.max_len;
  st.pos = st.ok ? static_cast<int>(pos) : 0;
  const int S = p.n_sink, W = p.window;
  st.new_full = st.pos < S || W > 0;
  st.new_in = st.ok && (st.new_full || live);
  st.leave_in = st.ok && live && W > 0 && st.pos - W >= S;
  st.to_ring = st.ok && st.new_full;
  st.slot = st.pos < S ? st.pos : (W > 0 ? S + (st.pos - S) % W : 0);
  st.mid_row = st.leave_in ? st.pos - W - S : (st.ok && live && !st.new_full ? st.pos - S : -1);
  return st;
}

// Element offsets of middle row r of head hd in batch row b: its K row and
// the V block that holds it (bf16 middle, paged or not).
__device__ __forceinline__ void middle_row_at(const DecodeParams& p, const DecodeHead& hd, int b,
                                              int64_t r, const uint16_t** k_row,
                                              const uint16_t** v_block) {
  if (p.paged) {
    const int64_t page = p.block_table[static_cast<int64_t>(b) * p.pages_per_row + r / LEANK_PAGE_ROWS];
    const uint16_t* base = p.pool + page * p.page_elems;
    const int64_t in = r % LEANK_PAGE_ROWS;
    *k_row = base + hd.k_off + in * hd.kept;
    *v_block = base + hd.v_off + (in / LEANK_V_BLOCK) * (LEANK_HEAD_DIM * LEANK_V_BLOCK);
  } else {
    *k_row = p.k_prun + hd.k_off + (static_cast<int64_t>(b) * p.mid_cap + r) * hd.kept;
    *v_block = p.v_mid + hd.v_off + static_cast<int64_t>(b) * p.v_mid_rows * LEANK_HEAD_DIM +
               (r / LEANK_V_BLOCK) * (LEANK_HEAD_DIM * LEANK_V_BLOCK);
  }
}

// Word `lane` of a token's compacted K row (kept channels 2 lane, 2 lane + 1
// of the head) from its full row in LDS.
__device__ __forceinline__ uint32_t compact_from_lds(const uint16_t* row, const int16_t* s_idx,
                                                     int kept, int lane) {
  const int j0 = 2 * lane;
  if (j0 >= kept) return 0u;
  return static_cast<uint32_t>(row[s_idx[j0] & (LEANK_HEAD_DIM - 1)]) |
         (static_cast<uint32_t>(row[s_idx[j0 + 1] & (LEANK_HEAD_DIM - 1)]) << 16);
}

}  // namespace leank
