/*
 * leank.h -- C ABI of the MI355X (gfx950) library for single-token decode
 * attention over a statically channel-pruned KV cache (LeanK style).
 *
 * The method is described on the page "大型语言模型KV缓存优化与LeanK剪枝技术解析"
 * (framerc.cn), called "the LeanK page" below:
 *   - section 2.2, stage 2: a binary channel mask from a learned importance
 *     alpha -- one global percentile threshold, a per-head count floored to
 *     a hardware alignment, then the top channels of each head;
 *   - section 3.1 items 1-3: heads grouped by kept-channel count, a
 *     full-width cache for the sink and local-window tokens, a compacted
 *     cache (K_prun) for the middle of the context, and one fused
 *     attention pass that loads only the kept channels;
 *   - section 3.2: a head with every channel pruned needs no middle V.
 * Grouped-query attention (a group of query heads shares one KV head) is as
 * in section 5.2.3 of "智能剪枝深度解析：大型语言模型KV缓存优化技术白皮书"; the
 * softmax scale convention Softmax(QK^T / sqrt(d)) is section 5.3 of the
 * FastGen page (mhpn.cn).
 *
 * Conventions for every entry point:
 *   - All buffers are caller-owned.  The library allocates no device memory
 *     and keeps no state between calls; every function is re-entrant.  The
 *     one exception is leank_decode_step_noalloc, for callers that cannot
 *     allocate: it uses a scratch array the library holds on each device.
 *   - "device" pointers address HIP device memory of the current device;
 *     "host" pointers address ordinary host memory.
 *   - bf16 tensors are passed as raw 16-bit patterns (void*).
 *   - Argument checks run on the host before any launch and return a
 *     negative leank_status; nothing is written then.  A failed launch or
 *     HIP call returns LEANK_EHIP.  No C++ exception crosses this boundary.
 *   - Asynchronous entry points enqueue work on `stream` (a hipStream_t
 *     passed as void*, NULL = the null stream) and return immediately.
 */
#ifndef LEANK_H
#define LEANK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LEANK_ABI_VERSION 7
#define LEANK_HEAD_DIM 128      /* the only head_dim the kernels implement   */
#define LEANK_MAX_KV_HEADS 64   /* per-layer KV heads a cache plan can hold  */
#define LEANK_MAX_GROUP 8       /* query heads per KV head the kernels take  */
#define LEANK_CHANNEL_QUANTUM 8 /* kept counts must be multiples of this     */
#define LEANK_V_BLOCK 8         /* V rows per transposed storage block        */
#define LEANK_QUANT_GROUP 64    /* middle rows per K quantization group       */
#define LEANK_PAGE_ROWS 64      /* middle rows per page of a paged cache      */
#define LEANK_NOALLOC_SCRATCH_BYTES (16u << 20) /* scratch of leank_decode_step_noalloc */

typedef enum {
  LEANK_OK = 0,
  LEANK_EINVAL = -1,        /* null pointer, size out of range, misaligned buffer, NaN in alpha */
  LEANK_EUNSUPPORTED = -2,  /* valid request outside what the kernels implement */
  LEANK_ECAPACITY = -3,     /* a position or context length beyond max_ctx */
  LEANK_EWORKSPACE = -4,    /* workspace missing or smaller than leank_workspace_bytes() */
  LEANK_EHIP = -5           /* a HIP runtime call or kernel launch failed */
} leank_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* leank_status_string(int status);

/* LEANK_ABI_VERSION of the built library. */
int leank_abi_version(void);

/* sizeof(leank_layer_cache) of the built library (lets bindings check their mirror). */
size_t leank_layer_cache_size(void);

/*
 * leank_build_mask -- the stage-2 mask of the LeanK page, section 2.2.
 *
 * alpha       device, float32 [n_layers][n_kv_heads][head_dim], finite or
 *             +-inf (NaN -> LEANK_EINVAL).  -0.0 and +0.0 compare equal.
 * prune_pct   prune ratio in percent, 0..100.  The global threshold is the
 *             order statistic of all n = n_layers*n_kv_heads*head_dim
 *             values at ascending rank ceil((n-1)*prune_pct/100), which is
 *             the set a linear-interpolation percentile selects; channels
 *             with alpha >= threshold pass the global step.
 * align       divides head_dim (LEANK_EINVAL otherwise) and is a multiple
 *             of LEANK_CHANNEL_QUANTUM (LEANK_EUNSUPPORTED otherwise: the
 *             cache plan takes kept counts in that quantum).  Each head's
 *             passing count is floored to a multiple of align; that many
 *             channels with the largest alpha of the head are kept, ties
 *             towards the lower channel index.
 * mask_out        device, uint8 [L][H][d]: 1 = kept.
 * kept_count_out  device, int32 [L][H]: kept channels per head.
 * kept_idx_out    device, int16 [L][H][d]: kept channel ids in ascending
 *                 order, then -1 padding.
 *
 * Runs two kernels on `stream` and waits for them (the threshold is read
 * back to the host between them through kept_count_out[0]); returns only
 * after the outputs are complete.  Host-side cost is one 4-byte copy.
 */
int leank_build_mask(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                     int32_t head_dim, int32_t prune_pct, int32_t align,
                     uint8_t* mask_out, int32_t* kept_count_out,
                     int16_t* kept_idx_out, void* stream);

/*
 * leank_build_mask_host -- the same mask from host memory, computed on the
 * host: the offline one-off conversion of the LeanK page, section 2.2
 * stage 2, for a caller that holds alpha on the host.  Host, synchronous,
 * pure; every pointer is host memory (alpha as above; mask_out uint8
 * [L][H][d], kept_count_out int32 [L][H], kept_idx_out int16 [L][H][d]).
 * Same rule, arguments and errors as leank_build_mask, and bit for bit the
 * same outputs.  Uses no device.
 */
int leank_build_mask_host(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                          int32_t head_dim, int32_t prune_pct, int32_t align,
                          uint8_t* mask_out, int32_t* kept_count_out, int16_t* kept_idx_out);

/*
 * One layer's channel-pruned KV cache: shape, head grouping and buffer
 * layout.  leank_plan_layer fills every field above `kept_idx`; the caller
 * allocates the four cache buffers with at least the *_bytes reported and
 * sets the pointers.  Layout (bf16 elements):
 *
 *   k_sl        [batch][n_kv_heads][n_sink + window][128], row-major:
 *               full-width keys of the sink and local-window tokens (LeanK
 *               page, section 3.1 item 2).  Token p < n_sink lives in row p;
 *               a window token p >= n_sink in ring row
 *               n_sink + (p - n_sink) % window.
 *   v_sl        [batch][n_kv_heads][V(n_sink + window)] with the same rows,
 *               stored in V blocks (below).
 *   k_prun      per live head h, at element offset k_prun_off[h]:
 *               [batch][mid_capacity][kept_count[h]], row-major --
 *               middle-of-context keys reduced to the kept channels, in
 *               ascending channel order; middle token p is row p - n_sink.
 *   v_mid       per live head h, at element offset v_mid_off[h]:
 *               [batch][V(mid_capacity)] middle values in V blocks.  Fully
 *               pruned heads have no segment (LeanK page, section 3.2).
 *
 * V blocks: a region of R rows x 128 channels takes ceil(R / 8) blocks of
 * 128 x 8 elements; element (row r, channel c) sits at
 * ((r / 8) * 128 + c) * 8 + r % 8, so each 16-byte piece holds 8
 * consecutive rows of one channel (the operand layout of the decode
 * kernel's matrix instructions).  V(R) denotes that storage, 128 * 8 *
 * ceil(R / 8) elements.
 *
 * Live heads are grouped by kept count (descending, then head id): their
 * segments follow `group_order`, so heads of one width form one contiguous
 * region (LeanK page, section 3.1 item 1).
 *
 * Low-bit middle streams (leank_plan_layer_q, quant_bits 4 or 8; LeanK page
 * section 4.2 and its deployment notes: quantize after prune and
 * reorganise; white paper section 5.2.1: INT8/INT4 codes, KIVI's per-channel
 * K and per-token V).  The middle of a live head is then held in five
 * buffers instead of k_prun / v_mid (k_prun_bytes = v_mid_bytes = 0):
 *
 *   k_q      per live head at byte offset k_q_off[h]: codes of the complete
 *            K groups, row-major [batch][G64][kept_count[h]] (G64 =
 *            ceil(mid_capacity / 64) * 64 rows); 4-bit codes two per byte,
 *            channel 2i in the low nibble of byte i.
 *   k_qp     per live head at float offset k_qp_off[h]: float32
 *            [batch][G64 / 64][kept_count[h]][2] = (scale, minimum) of each
 *            channel over each group of 64 middle rows.
 *   k_stage  per live head at element offset k_stage_off[h]: bf16
 *            [batch][64][kept_count[h]], the rows of the group that is not
 *            complete yet (middle row r in stage row r % 64).
 *   v_q      per live head at byte offset v_q_off[h]: V codes in 8-row blocks
 *            [batch][ceil(mid_capacity / 8)][128][8 codes]: 8-bit, byte
 *            ((r / 8) * 128 + c) * 8 + r % 8; 4-bit, 4 bytes per (block,
 *            channel), byte k holding row k (low nibble) and k + 4.
 *   v_qp     per live head at float offset v_qp_off[h]: float32
 *            [batch][mid_capacity][2] = (scale, minimum) of each middle row.
 *
 * A value is code * scale + minimum.  Codes: minimum and scale = (max -
 * min) / (2^bits - 1) of the group, code = round-half-even((x - min) /
 * scale) clamped to [0, 2^bits - 1] (0 when scale is 0), decided in IEEE
 * float32.  K and V must be finite.  Sink and window rows stay bf16.
 *
 * Paged middle (leank_plan_layer_paged; white paper section 3, block-level
 * granularity: the cache of a serving system such as vLLM's PagedAttention
 * is organised in fixed-size blocks; its worked example block holds 64
 * tokens).  The middle rows of batch row b are held in pages of
 * LEANK_PAGE_ROWS rows taken from a caller-owned pool: middle row r lives
 * in physical page block_table[b * pages_per_row + r / 64], row r % 64 of
 * it.  One page holds those 64 rows for every live head: first, head by
 * head in group order, K as [64][kept_count[h]] at element offset
 * k_prun_off[h]; then, head by head, V as 8 V blocks [8][128][8] at element
 * offset v_mid_off[h] (element offsets within the page; bf16).  k_prun and
 * v_mid are unused (k_prun_bytes = v_mid_bytes = 0).  The caller maps a
 * page before rows are appended to it (for one token per step: whenever
 * r % 64 == 0); the kernels read the table on the device and do not check
 * it, so every entry that covers written rows must lie in [0, n_pages),
 * and distinct entries (of any batch row) must name distinct pages.
 *
 * Paged low-bit middle (leank_plan_layer_paged_q): a page holds one 64-row
 * K group of every live head.  Within the page, at byte offsets: the K
 * codes of the live heads in group order, each [64][kept_count[h]] at
 * k_q_off[h]; then their K (scale, minimum) pairs, float32
 * [kept_count[h]][2] at float offset k_qp_off[h]; then their V codes, 8
 * blocks as in v_q at v_q_off[h]; then their V row parameters, float32
 * [64][2] at float offset v_qp_off[h].  The staging rows of the open group
 * stay in k_stage; k_q, k_qp, v_q and v_qp are unused (their sizes are 0).
 */
typedef struct leank_layer_cache {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_sink;
  int32_t window;
  int64_t max_ctx;        /* tokens the cache can hold */
  int64_t mid_capacity;   /* max(0, max_ctx - n_sink - window) */
  int32_t n_live;         /* heads with kept_count > 0 */
  int32_t reserved0;
  int32_t kept_count[LEANK_MAX_KV_HEADS];
  int32_t group_order[LEANK_MAX_KV_HEADS];  /* live heads by (count desc, id asc), then dead */
  int64_t k_prun_off[LEANK_MAX_KV_HEADS];   /* elements; -1 for dead heads */
  int64_t v_mid_off[LEANK_MAX_KV_HEADS];    /* elements; -1 for dead heads */
  uint64_t k_sl_bytes;
  uint64_t v_sl_bytes;
  uint64_t k_prun_bytes;
  uint64_t v_mid_bytes;
  /* set by the caller: */
  const int16_t* kept_idx; /* device int16 [n_kv_heads][128], as leank_build_mask writes it */
  void* k_sl;              /* device, 16-byte aligned */
  void* v_sl;
  void* k_prun;
  void* v_mid;
  /* low-bit middle streams (filled by leank_plan_layer_q; zero otherwise) */
  int32_t quant_bits;                        /* 0 (bf16 middle), 4 or 8 */
  int32_t quant_group;                       /* LEANK_QUANT_GROUP, or 0 */
  int64_t k_q_off[LEANK_MAX_KV_HEADS];       /* bytes; -1 for dead heads */
  int64_t k_qp_off[LEANK_MAX_KV_HEADS];      /* floats; -1 for dead heads */
  int64_t k_stage_off[LEANK_MAX_KV_HEADS];   /* elements; -1 for dead heads */
  int64_t v_q_off[LEANK_MAX_KV_HEADS];       /* bytes; -1 for dead heads */
  int64_t v_qp_off[LEANK_MAX_KV_HEADS];      /* floats; -1 for dead heads */
  uint64_t k_q_bytes;
  uint64_t k_qp_bytes;
  uint64_t k_stage_bytes;
  uint64_t v_q_bytes;
  uint64_t v_qp_bytes;
  /* set by the caller (16-byte aligned) when quant_bits != 0: */
  void* k_q;
  void* k_qp;
  void* k_stage;
  void* v_q;
  void* v_qp;
  /* paged middle (filled by leank_plan_layer_paged; zero otherwise) */
  int32_t page_rows;            /* LEANK_PAGE_ROWS, or 0 */
  int32_t pages_per_row;        /* block table entries per batch row: ceil(mid_capacity / 64) */
  int64_t n_pages;              /* pages in the pool */
  uint64_t page_bytes;          /* 64 * sum over live heads of (2 * kept_count + 256) */
  uint64_t pool_bytes;          /* n_pages * page_bytes */
  /* set by the caller when page_rows != 0: */
  void* pool;                   /* device, 16-byte aligned */
  const int32_t* block_table;   /* device int32 [batch][pages_per_row] */
} leank_layer_cache;

/*
 * leank_plan_layer -- host, pure.  kept_count_host: host int32
 * [n_kv_heads] (one layer's row of kept_count_out).  Requirements:
 * head_dim == 128; 1 <= n_kv_heads <= LEANK_MAX_KV_HEADS; n_q_heads a
 * multiple of n_kv_heads with n_q_heads / n_kv_heads <= LEANK_MAX_GROUP;
 * every kept count in [0, 128] and a multiple of LEANK_CHANNEL_QUANTUM
 * (LEANK_EUNSUPPORTED otherwise); batch >= 1; n_sink, window >= 0 with
 * n_sink + window >= 1 (so every head always has a full-width token);
 * max_ctx >= 1.  Clears the caller-set pointer fields.
 */
int leank_plan_layer(const int32_t* kept_count_host, int32_t batch,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int32_t n_sink, int32_t window, int64_t max_ctx,
                     leank_layer_cache* cache_out);

/*
 * leank_plan_layer_q -- leank_plan_layer for a cache whose middle is held
 * in low-bit streams (quant_bits 4 or 8; 0 gives the bf16 plan).  Same
 * requirements; the caller allocates k_sl, v_sl and the five low-bit
 * buffers.  Every entry point works on such a cache.  leank_pack_k packs a
 * prefill into an empty cache (pos0 == 0) in bulk and takes any other
 * append, like leank_pack_k_rows, token by token in one kernel (a token
 * that completes a K group quantizes the group).  leank_decode_step fuses
 * the append into the attention except when the row it moves to the
 * middle completes a K group, and leank_decode_step_rows always runs the
 * append first: both then launch the append kernel before the two decode
 * kernels.  In the ragged decode calls ctx_lens[b] / row_pos[b] must be
 * the row's current length, since its open K group is staged for that
 * length.
 */
int leank_plan_layer_q(const int32_t* kept_count_host, int32_t batch,
                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                       int32_t n_sink, int32_t window, int64_t max_ctx,
                       int32_t quant_bits, leank_layer_cache* cache_out);

/*
 * leank_plan_layer_paged -- leank_plan_layer for a bf16 cache whose middle
 * is held in pages of 64 rows from a pool of n_pages pages (n_pages >= 1)
 * through a block table (layout above).  max_ctx bounds every batch row.
 * The caller allocates k_sl, v_sl, the pool (pool_bytes) and the block
 * table (int32 [batch][pages_per_row]).  Every entry point takes such a
 * cache.
 */
int leank_plan_layer_paged(const int32_t* kept_count_host, int32_t batch,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           int32_t n_sink, int32_t window, int64_t max_ctx,
                           int64_t n_pages, leank_layer_cache* cache_out);

/*
 * leank_plan_layer_paged_q -- a cache whose middle is both low-bit
 * (quant_bits 4 or 8, as leank_plan_layer_q) and paged (as
 * leank_plan_layer_paged; page layout above).  quant_bits 0 gives
 * leank_plan_layer_paged.  The caller allocates k_sl, v_sl, k_stage, the
 * pool and the block table.  Every entry point takes such a cache, with the
 * low-bit rules of leank_plan_layer_q.
 */
int leank_plan_layer_paged_q(const int32_t* kept_count_host, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                             int32_t n_sink, int32_t window, int64_t max_ctx,
                             int64_t n_pages, int32_t quant_bits,
                             leank_layer_cache* cache_out);

/*
 * leank_pack_k -- append n_new tokens at positions [pos0, pos0 + n_new)
 * (LeanK page, section 3.1 item 2).  pos0 must equal the number of tokens
 * already in the cache (append-only; the library does not track it).
 *
 * k_new, v_new  device bf16 [batch][n_kv_heads][n_new][128].
 *
 * Sink tokens go to their rows of k_sl/v_sl.  Window tokens go to their
 * ring rows; a token that the append pushes out of the window is first
 * moved to the middle: its kept K channels gathered into k_prun and its V
 * row copied into v_mid (dropped for fully pruned heads).  New tokens that
 * are already out of the window when the append ends go straight to the
 * middle.  Bit copies only.  Errors: LEANK_ECAPACITY if pos0 + n_new >
 * max_ctx.  n_new == 0 is a no-op.  One kernel when n_new <= window, two
 * otherwise; asynchronous on `stream`.
 */
int leank_pack_k(const leank_layer_cache* cache, const void* k_new,
                 const void* v_new, int64_t pos0, int64_t n_new, void* stream);

/*
 * leank_workspace_bytes -- host.  Bytes of device workspace
 * leank_decode_attn (and its ragged form) needs for a context of ctx_len
 * tokens, which also covers a fused step (leank_decode_step and its ragged
 * form) whose context after the append is ctx_len.  Non-decreasing in
 * ctx_len, so the size for max_ctx serves every call.
 */
int leank_workspace_bytes(const leank_layer_cache* cache, int64_t ctx_len,
                          size_t* bytes_out);

/*
 * leank_workspace_init -- zero-fill a workspace (optional: leank_decode_attn
 * writes every workspace byte it later reads, so a fresh workspace needs
 * no preparation).  Asynchronous on `stream` (a fill kernel, no memset
 * node).  workspace_bytes must be a multiple of 4.
 */
int leank_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * leank_decode_attn -- one decode step of attention for every (batch row,
 * query head) of one layer (LeanK page, section 3.1 item 3 and section
 * 3.2).
 *
 * q         device bf16 [batch][n_q_heads][128]; query head j reads KV
 *           head j / (n_q_heads / n_kv_heads).
 * ctx_len   tokens in the cache (1..max_ctx), newest included.
 * scale     softmax scale, normally 1/sqrt(128).
 * out       device float32 [batch][n_q_heads][128].
 *
 * For query head j of KV head h, over the cached tokens t:
 *   score(t) = scale * q_j . K[t]            sink and window tokens,
 *   score(t) = scale * sum_i q_j[idx_h[i]] K_prun[t][i]
 *                                            middle tokens of a live head,
 *   middle tokens of a fully pruned head take no part;
 *   out_j = sum_t softmax(score)_t V[t].
 * bf16 inputs, float32 accumulation.  q and the cache must be finite: the
 * output for a NaN or infinite input is unspecified.  The context is split
 * into work items whose partial (max, sum, weighted V) records go to the
 * workspace; a second kernel merges each (batch row, KV head) pair's records
 * in a fixed order, so the output does not depend on scheduling.  Two kernel
 * launches, asynchronous on `stream`.  Calls that share a workspace must not
 * overlap in time.
 */
int leank_decode_attn(const leank_layer_cache* cache, const void* q,
                      int64_t ctx_len, float scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged batches (rows at different context lengths).
 *
 * leank_pack_k_rows -- like leank_pack_k, but batch row b appends
 *   row_count[b] tokens (tokens [0, row_count[b]) of its slice of k_new /
 *   v_new, bf16 [batch][n_kv_heads][n_new][128]) at positions
 *   [row_pos[b], row_pos[b] + row_count[b]).  row_pos: device int64
 *   [batch], the row's current length; row_count: device int32 [batch]
 *   with values in [0, n_new], or NULL for n_new everywhere.  The arrays
 *   are read on the device, so they are not validated on the host: a row
 *   whose positions fall outside [0, max_ctx] is left unchanged.  One
 *   kernel when n_new <= window, two otherwise; asynchronous on `stream`.
 *
 * leank_decode_attn_rows -- like leank_decode_attn, with batch row b
 *   attending over its first ctx_lens[b] tokens (device int32 [batch],
 *   values clamped to [0, max_ctx_len]); max_ctx_len (1..max_ctx) sizes the
 *   work plan and the workspace.  A row of length 0 gets a zero output.
 */
int leank_pack_k_rows(const leank_layer_cache* cache, const void* k_new, const void* v_new,
                      const int64_t* row_pos, const int32_t* row_count, int64_t n_new,
                      void* stream);
int leank_decode_attn_rows(const leank_layer_cache* cache, const void* q,
                           const int32_t* ctx_lens, int64_t max_ctx_len, float scale,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused decode step: the append of one token per batch row and the decode
 * attention that follows it, in the two kernels of leank_decode_attn.
 *
 * leank_decode_step -- same result as leank_pack_k(cache, k_new, v_new,
 *   pos, 1) followed by leank_decode_attn(cache, q, pos + 1, ...): the
 *   cache afterwards holds bit for bit what that append writes (LeanK page,
 *   section 3.1 item 2: the token leaving the window moves its kept K
 *   channels and, for a live head, its V to the middle), and out holds the
 *   attention of q over the pos + 1 tokens (section 3.1 item 3, 3.2).
 *   k_new, v_new: device bf16 [batch][n_kv_heads][128] (16-byte aligned),
 *   the token at position pos = the cache's current length (0..max_ctx-1;
 *   pos + 1 > max_ctx -> LEANK_ECAPACITY).  q, scale, out, workspace as in
 *   leank_decode_attn; the workspace needs leank_workspace_bytes(cache,
 *   pos + 1) bytes.  No cache row is written before every read of it in
 *   the call is done, so the step is safe without any extra ordering.
 *
 * leank_decode_step_rows -- the same with batch row b appending at its own
 *   position row_pos[b] (device int64 [batch], the row's current length)
 *   and attending over row_pos[b] + 1 tokens.  max_ctx_len (1..max_ctx)
 *   bounds row_pos[b] + 1 and sizes the work plan and the workspace
 *   (leank_workspace_bytes(cache, max_ctx_len)).  row_pos is read on the
 *   device: a row with row_pos[b] outside [0, max_ctx_len - 1] is left
 *   unchanged and gets a zero output.
 */
int leank_decode_step(const leank_layer_cache* cache, const void* q, const void* k_new,
                      const void* v_new, int64_t pos, float scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);
int leank_decode_step_rows(const leank_layer_cache* cache, const void* q, const void* k_new,
                           const void* v_new, const int64_t* row_pos, int64_t max_ctx_len,
                           float scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * leank_decode_step_noalloc -- leank_decode_step for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments and result as
 * leank_decode_step without the workspace: the split-K records go to a
 * scratch array of LEANK_NOALLOC_SCRATCH_BYTES that the library holds on
 * each device it runs on, from that device's first call until the process
 * ends.  Allocates nothing (no hipMalloc, hipFree or allocating library
 * call); the first call on a device looks the array's address up.
 * Errors: as leank_decode_step, and LEANK_EWORKSPACE, before any launch,
 * when the call needs more than LEANK_NOALLOC_SCRATCH_BYTES
 * (leank_workspace_bytes(cache, pos + 1) larger).  Every call on a device
 * shares that device's array: calls that overlap in time on one device
 * (other streams, other threads) race and must be serialised by the
 * caller.
 */
int leank_decode_step_noalloc(const leank_layer_cache* cache, const void* q, const void* k_new,
                              const void* v_new, int64_t pos, float scale, float* out,
                              void* stream);

/*
 * leank_decode_bytes -- host.  Algorithmic HBM bytes of one
 * leank_decode_attn call: q (bf16) + full-width K and V of every head +
 * kept K channels and V of live heads over the middle + out (float32).
 * The split-K workspace traffic is not counted.
 */
int leank_decode_bytes(const leank_layer_cache* cache, int64_t ctx_len,
                       int64_t* bytes_out);

/*
 * Analysis helpers (host, synchronous, pure; host pointers).  Offline tools
 * over alpha and masks, from the LeanK page's section 6 (which channel
 * pairs and heads the learned importance keeps) and section 2.1 (the
 * channel-importance ranking is stable across tasks and lengths).  Channel
 * pair i joins channels i and i + head_dim/2 (rotate-half RoPE pairing); a
 * lower pair index is a higher rotary frequency.
 *
 * leank_pair_retention -- retention_out[i], i < head_dim/2: mean over the
 *   n_layers*n_kv_heads rows of mask (uint8 [L][H][d]) of
 *   (kept(i) + kept(i + d/2)) / 2.
 * leank_head_hf_ratio -- w_hf_out[l*H + h]: share of the row's |alpha| mass
 *   on its n_hf_pairs highest-frequency pairs (0 for an all-zero row).
 *   NaN in alpha -> LEANK_EINVAL.
 * leank_rank_correlation -- Pearson correlation of two alpha arrays of n
 *   values, and Pearson correlation of their ranks (equal values get the
 *   mean of the ranks they span).  n >= 2; NaN -> LEANK_EINVAL; a constant
 *   input gives 0.
 */
int leank_pair_retention(const uint8_t* mask, int32_t n_layers, int32_t n_kv_heads,
                         int32_t head_dim, double* retention_out);
int leank_head_hf_ratio(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                        int32_t head_dim, int32_t n_hf_pairs, double* w_hf_out);
int leank_rank_correlation(const float* a, const float* b, int64_t n, double* pearson_out,
                           double* rank_pearson_out);

#ifdef __cplusplus
}
#endif

#endif /* LEANK_H */
