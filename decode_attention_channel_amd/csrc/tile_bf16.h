// Tiles of bf16 streams: the full-width sink and window rows and the
// bf16 middle (contiguous or paged).  A wavefront takes 32-row tiles
// round-robin; per tile it loads K (16-byte rows) and V (8-row blocks),
// forms the scores and the weights and accumulates P V with the matrix
// instructions.
#pragma once

#include "decode_base.h"

namespace leank {

// K and V operands of one 32-row tile.
template <int KB>
struct TileRegs {
  u32x4_t kf[2][KB];  // K rows t0 + 16 j + col, channels 32 kk + 8 grp .. +7
  u32x4_t vf[8];      // V block t0 / 8 + grp, channel 16 n + col
};

// Scores, softmax bookkeeping and weighted V of one loaded tile.  The
// masked variant (kTail) drops rows >= nvalid and row excl_rel (a ring row
// that a fused step replaces; any value outside [0, 32) drops nothing).
template <int G, int KB, bool kTail>
__device__ __forceinline__ void compute_tile(TileRegs<KB>& tr, int nvalid, int excl_rel,
                                             const u32x4_t (&qa)[KB],
                                             float qk_scale, uint16_t* __restrict__ p_lds,
                                             WaveState& st) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;

  // scores: s[j][i] = head 4 grp + i, row 16 j + col
  f32x4_t s[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    s[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) s[j] = mfma_bf16(qa[kk], tr.kf[j][kk], s[j]);
  }

  float mx[4];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v = s[j][i] * qk_scale;
      if (kTail && (16 * j + col >= nvalid || 16 * j + col == excl_rel)) v = -INFINITY;
      s[j][i] = v;
    }
    mx[i] = fmaxf(s[0][i], s[1][i]);  // this lane's rows
    grow |= mx[i] > st.m[i] + kRescaleSlack;
  }
  // a head's tile maximum passes its reference by more than the slack iff
  // one of its lanes does, so the row reductions run only then
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float tile_max = row_max16(mx[i]);
      float corr = 1.0f;
      if (tile_max > st.m[i] + kRescaleSlack) {
        corr = st.m[i] == -INFINITY ? 0.0f : fast_exp2(st.m[i] - tile_max);
        st.m[i] = tile_max;
      }
      st.l[i] *= corr;
#pragma unroll
      for (int n = 0; n < 8; ++n) st.o[n][i] *= corr;
    }
  }

  // weights, staged in LDS as bf16 hi/lo parts: p_lds[part][head][row]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m_use = st.m[i] == -INFINITY ? 0.0f : st.m[i];
    const int head = 4 * grp + i;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float p = fast_exp2(s[j][i] - m_use);
      st.l[i] += p;
      // every head's row is written (rows of heads >= G only feed output
      // rows that are never recorded), so the stores need no branch
      const __bf16 hi = static_cast<__bf16>(p);
      const __bf16 lo = static_cast<__bf16>(p - static_cast<float>(hi));
      p_lds[head * kTileRows + 16 * j + col] = __builtin_bit_cast(uint16_t, hi);
      p_lds[(16 + head) * kTileRows + 16 * j + col] = __builtin_bit_cast(uint16_t, lo);
    }
  }
  const u32x4_t pa_hi = *reinterpret_cast<const u32x4_alias_t*>(p_lds + col * kTileRows + 8 * grp);
  const u32x4_t pa_lo = *reinterpret_cast<const u32x4_alias_t*>(p_lds + (16 + col) * kTileRows + 8 * grp);

  if (kTail) {
    // zero the V rows of the lane's block that are dropped
    u32x4_t keep;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e0 = 8 * grp + 2 * w, e1 = e0 + 1;
      keep[w] = (e0 < nvalid && e0 != excl_rel ? 0x0000ffffu : 0u) |
                (e1 < nvalid && e1 != excl_rel ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) tr.vf[n] &= keep;
  }

#pragma unroll
  for (int n = 0; n < 8; ++n) {
    st.o[n] = mfma_bf16(pa_hi, tr.vf[n], st.o[n]);
    st.o[n] = mfma_bf16(pa_lo, tr.vf[n], st.o[n]);
  }
}

// Buffer resource over `bytes` bytes from `base` (both the same in every
// lane of the wavefront): a load at or past the end returns zeros and
// touches no memory.  The values go through readfirstlane so that the
// descriptor sits in scalar registers even where they derive from vector
// loads (a ragged row's length).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const uint16_t* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int nb = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes > 0 ? bytes : 0));
  return __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0, nb, kRsrcWord3);
}

// 16-byte streaming load through a buffer resource (cache data read once
// per call: non-temporal, as load_stream16).
__device__ __forceinline__ u32x4_t load_buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNT));
  return v;
}

// load_tile over the rows of one item: rk holds the item's K rows (kstride
// elements each) from its first row, rv its V blocks; t is the tile's
// first row counted from the item's first row.  Rows past the item and
// channels past c come back as zeros from the resources' bounds, so no lane
// branches.
template <int KB>
__device__ __forceinline__ void load_tile_buf(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                              int kstride, int t, int c, TileRegs<KB>& tr) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const uint32_t k0 = static_cast<uint32_t>(((t + col) * kstride + 8 * grp) * 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const uint32_t off = k0 + static_cast<uint32_t>((16 * j * kstride + 32 * kk) * 2);
      tr.kf[j][kk] = load_buf16(rk, 32 * kk + 8 * grp < c ? off : kBufOutside);
    }
  }
  const uint32_t v0 = static_cast<uint32_t>(((t / 8 + grp) * LEANK_HEAD_DIM + col) * 16);
#pragma unroll
  for (int n = 0; n < 8; ++n) tr.vf[n] = load_buf16(rv, v0 + n * 256);
}

// Rows [r0, r1) of one stream, except row excl (-1: none).  `stage` issues
// the workgroup's staging loads (q rows and kept ids; the caller defines
// it) and returns the part that writes them to LDS; each wavefront issues
// its first tile's loads in between, then writes its part of the staging,
// joins the workgroup barrier that publishes it and gathers its query
// operand, so the two memory latencies at the start of an item overlap.
// (Issuing the staging loads after the tile's, so that they return behind
// them, measured slower: the Llama batch-64 4K step 110.9 -> 112.7 us, the
// 32-layer 128K-token batch-1 token 960 -> 970 us.)  The loads go through
// buffer resources bounded by the item's rows, so the last tile needs no
// lane branches (measured against per-lane predicated global loads: the
// 32-layer 128K-token batch-1 token 991 -> 978 us, the Qwen2.5-7B-shaped
// batch-16 32K step 90.1 -> 89.4 us).  Keeping a second tile in flight per
// wavefront (two tiles of registers, so two workgroups per compute unit
// instead of three) measured slower: 1051 us and 98 us.  Every thread of
// the workgroup must call this (it holds the barrier).
template <int G, int KB, class Stage>
__device__ __forceinline__ void attend_range_staged(const uint16_t* kb, int kstride,
                                                    const uint16_t* vb, int r0, int r1, int excl,
                                                    int c, const uint16_t* s_q,
                                                    const int16_t* s_idx, bool dense,
                                                    float qk_scale, uint16_t* p_lds,
                                                    WaveState& st, Stage&& stage) {
  constexpr int kStep = kWaves * kTileRows;
  const int wave = threadIdx.x >> 6;
  const int n = r1 - r0;  // rows of the item (r0 is a multiple of 8)
  const __amdgpu_buffer_rsrc_t rk = stream_rsrc(kb + static_cast<int64_t>(r0) * kstride,
                                                static_cast<int64_t>(n) * kstride * 2);
  const __amdgpu_buffer_rsrc_t rv =
      stream_rsrc(vb + static_cast<int64_t>(r0 / 8) * (LEANK_HEAD_DIM * 8),
                  static_cast<int64_t>((n + 7) / 8) * (LEANK_HEAD_DIM * 8 * 2));
  const int ex = excl < 0 ? -1 : excl - r0;
  int t = wave * kTileRows;
  TileRegs<KB> tr;
  const auto commit = stage();
  load_tile_buf<KB>(rk, rv, kstride, t, c, tr);
  commit();
  __syncthreads();
  u32x4_t qa[KB];
  gather_q<G, KB>(s_q, s_idx, dense, c, qa);
  while (t < n) {
    if (n - t >= kTileRows && static_cast<unsigned>(ex - t) >= kTileRows)
      compute_tile<G, KB, false>(tr, kTileRows, -1, qa, qk_scale, p_lds, st);
    else
      compute_tile<G, KB, true>(tr, n - t, ex - t, qa, qk_scale, p_lds, st);
    t += kStep;
    if (t < n) load_tile_buf<KB>(rk, rv, kstride, t, c, tr);
  }
}

// Middle rows [r0, r1) of a paged stream: r0 is a multiple of the page
// size and s_pages holds the physical pages of rows r0, r0 + 64, ...
// (tiles never straddle a page: both are 32-row aligned).  Each tile loads
// through resources over its page's rows that belong to the item.  Staged
// as attend_range_staged: the first tile's page comes from g_pages, the
// block table entries of the same rows in global memory, while s_pages and
// the q rows are still on their way to LDS.  Every thread of the workgroup
// must call this (it holds the barrier).
template <int G, int KB>
__device__ __forceinline__ void attend_range_paged_staged(
    const uint16_t* pool, int64_t page_elems, const int32_t* g_pages, const int32_t* s_pages,
    int64_t k_off, int64_t v_off, int r0, int r1, int c, const uint16_t* s_q,
    const int16_t* s_idx, float qk_scale, uint16_t* p_lds, WaveState& st) {
  constexpr int kStep = kWaves * kTileRows;
  const int wave = threadIdx.x >> 6;
  const int n = r1 - r0;
  // loads of the tile at item row t from physical page `page`
  auto load = [&](int t, int32_t page, TileRegs<KB>& tr) {
    const int in = t % LEANK_PAGE_ROWS;         // row within the page
    const int rows = min(LEANK_PAGE_ROWS, n - (t - in));  // the item's rows in the page
    const uint16_t* base = pool + static_cast<int64_t>(page) * page_elems;
    load_tile_buf<KB>(stream_rsrc(base + k_off, static_cast<int64_t>(rows) * c * 2),
                      stream_rsrc(base + v_off, static_cast<int64_t>((rows + 7) / 8) * (LEANK_HEAD_DIM * 8 * 2)),
                      c, in, c, tr);
  };
  int t = wave * kTileRows;
  TileRegs<KB> tr;
  if (t < n) load(t, __builtin_amdgcn_readfirstlane(g_pages[t / LEANK_PAGE_ROWS]), tr);
  __syncthreads();
  u32x4_t qa[KB];
  gather_q<G, KB>(s_q, s_idx, false, c, qa);
  while (t < n) {
    if (n - t >= kTileRows)
      compute_tile<G, KB, false>(tr, kTileRows, -1, qa, qk_scale, p_lds, st);
    else
      compute_tile<G, KB, true>(tr, n - t, -1, qa, qk_scale, p_lds, st);
    t += kStep;
    if (t < n) load(t, __builtin_amdgcn_readfirstlane(s_pages[t / LEANK_PAGE_ROWS]), tr);
  }
}

}  // namespace leank
