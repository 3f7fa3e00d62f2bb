"""Plain, slow CPU oracle for LeanK-style channel-pruned decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The product
(the HIP library and its Python binding) never does, and this module imports
nothing from the product: the two share no code.

Sources (cited by page title and section):

* LeanK page -- "大型语言模型KV缓存优化与LeanK剪枝技术解析" (framerc.cn):
  - section 1: KV-cache size is 2 x L x h x d x N elements;
  - section 2.2, stage 1: the learned scale alpha has shape L x h x d and is
    applied only to the middle of the context (not the sink tokens, not the
    sliding local window);
  - section 2.2, stage 2: the hardware-friendly mask -- one global
    percentile threshold over all of alpha, then per head the kept count is
    floored to the alignment and the top-k channels of that head are kept;
  - section 3.1, item 2: sink + local-window keys are stored full width,
    the middle of the context is stored channel-pruned;
  - section 3.1 (kernel sketch): only the kept channels are loaded;
  - section 3.2: a head whose channels are all pruned can drop its V cache.
* KV-pruning white paper -- "智能剪枝深度解析：大型语言模型KV缓存优化技术白皮书"
  (blog.yyx235.top): section 3.3.1 (attention sinks + sliding window),
  section 5.2.3 (grouped-query attention: a group of query heads shares one
  K/V head).
* FastGen page (mhpn.cn, FastGen / ICLR 2024): section 2.2 (worked KV-cache
  size example), section 5.3 (attention weights are Softmax(QK^T / sqrt(d))).

Readings taken where the pages are silent or garbled (each one is listed in
the design notes of the repository):

* prune_pct is the prune ratio of the prose; the threshold is the
  prune_pct-th percentile of alpha and channels with alpha >= threshold
  survive the global step.  The linear-interpolation percentile is replaced
  by the exact order statistic at rank ceil((N-1)*p/100), which selects the
  same channels (the interpolated value always lies strictly above the
  lower neighbour unless the two neighbours are equal);
* top-k ties are broken towards the lower channel index; kept channel ids
  are reported in ascending order;
* a query head j reads KV head j // G (contiguous GQA groups);
* a fully-pruned head excludes its middle tokens from the softmax (no
  weight, no V), it does not score them as zero;
* the softmax scale is 1/sqrt(head_dim) with the full head_dim;
* regions for a context of T tokens: sink [0, min(S, T)), local window
  [max(S, T - W), T), middle [S, T - W) (empty when T <= S + W);
* cache layout of the full-width region: sink token p < S in slot p, a
  window token p >= S in ring slot S + (p - S) mod W.

Low-bit middle streams (LeanK page, section 4.2 and its deployment notes:
quantization composes with the pruning and comes after prune and
reorganisation; white paper section 5.2.1: INT8/INT4 codes, per-channel K
and per-token V as in KIVI).  The pages give no formula; the reading taken:

* asymmetric uniform quantization over a group of values x: lo = min x,
  hi = max x, scale = (hi - lo) / (2^bits - 1), code = round-half-even of
  (x - lo) / scale clamped to [0, 2^bits - 1] (code 0 when scale = 0); the
  value represented is code * scale + lo;
* the code is an integer decided by floating point, so it is decided in
  IEEE float32 (one subtraction, one division, as written);
* K (the kept channels of the middle) is quantized per channel over groups
  of 64 consecutive middle rows of one (batch row, KV head); the rows of a
  group that is not yet complete stay bf16 until the group fills;
* V of the middle is quantized per token (one scale and minimum over the
  token's 128 channels);
* the sink and window rows stay bf16 (they play the part of KIVI's
  full-precision residual).

Every floating-point step runs in float64 on bf16 inputs widened exactly,
except the quantization decision above (float32).
"""

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "prune_rank",
    "build_mask",
    "regions",
    "ring_slot",
    "pack_reference",
    "decode",
    "decode_f64",
    "QUANT_GROUP",
    "quantize_asym",
    "dequantize",
    "quantize_middle",
    "pack_reference_q",
    "decode_q",
    "kv_cache_bytes",
    "decode_traffic_bytes",
    "decode_traffic_bytes_q",
    "pair_retention",
    "head_hf_ratio",
    "rank_correlation",
]


def bf16_bits_to_f64(bits):
    """Widen bf16 bit patterns (uint16) to float64 exactly.

    A bf16 value is the upper half of an IEEE float32; widening to float32
    and then float64 is exact.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def prune_rank(n, prune_pct):
    """Rank (0-based, ascending) of the global threshold among n values.

    LeanK page, section 2.2 stage 2: the threshold is a percentile of the
    flattened alpha.  With linear interpolation at position (n-1)*p/100, the
    set {alpha >= value} equals {alpha >= x[ceil((n-1)*p/100)]} for the
    ascending order statistics x, so the rank is that ceiling, taken in
    integer arithmetic.
    """
    return -((-(n - 1) * prune_pct) // 100)


def build_mask(alpha, prune_pct, align):
    """Stage-2 mask of the LeanK page, section 2.2.

    alpha: float32 array [L, H, d] (H = KV heads).
    Returns (mask uint8 [L, H, d], kept_count int32 [L, H],
             kept_idx int16 [L, H, d] -- ascending kept channels, -1 padded).

    Steps, in the page's order:
    1. one threshold over all of alpha: the prune_pct-th percentile;
    2. per (layer, head): count the channels with alpha >= threshold;
    3. floor that count to a multiple of `align`;
    4. keep that many channels with the largest alpha of the head
       (ties towards the lower channel index).
    """
    alpha = np.asarray(alpha)
    if alpha.dtype != np.float32 or alpha.ndim != 3:
        raise ValueError("alpha must be a float32 array [L, H, d]")
    if np.any(np.isnan(alpha)):
        raise ValueError("alpha holds NaN")
    n_layers, n_heads, d = alpha.shape
    if not 0 <= prune_pct <= 100:
        raise ValueError("prune_pct must lie in [0, 100]")
    if align < 1 or d % align != 0:
        raise ValueError("align must be >= 1 and divide head_dim")
    n = alpha.size
    if n == 0:
        raise ValueError("alpha is empty")

    values = alpha.astype(np.float64)
    ordered = np.sort(values.ravel())
    threshold = ordered[prune_rank(n, prune_pct)]

    mask = np.zeros((n_layers, n_heads, d), dtype=np.uint8)
    kept_count = np.zeros((n_layers, n_heads), dtype=np.int32)
    kept_idx = np.full((n_layers, n_heads, d), -1, dtype=np.int16)
    for layer in range(n_layers):
        for head in range(n_heads):
            a = values[layer, head]
            n_keep = int(np.count_nonzero(a >= threshold))
            n_keep = (n_keep // align) * align
            by_importance = sorted(range(d), key=lambda c: (-a[c], c))
            kept = sorted(by_importance[:n_keep])
            mask[layer, head, kept] = 1
            kept_count[layer, head] = n_keep
            kept_idx[layer, head, :n_keep] = kept
    return mask, kept_count, kept_idx


def regions(ctx_len, n_sink, window):
    """Split positions [0, ctx_len) into (sink, middle, local) ranges.

    LeanK page, section 2.2 stage 1 and section 3.1 item 2; white paper
    section 3.3.1.  Returns three Python ranges.
    """
    sink = range(0, min(n_sink, ctx_len))
    local_begin = max(n_sink, ctx_len - window)
    middle = range(n_sink, local_begin)
    local = range(local_begin, ctx_len)
    return sink, middle, local


def ring_slot(pos, n_sink, window):
    """Slot of a full-width token: sink tokens in place, window tokens in a ring."""
    if pos < n_sink:
        return pos
    return n_sink + (pos - n_sink) % window


def pack_reference(k_bits, v_bits, kept_count, kept_idx, n_sink, window):
    """Expected cache contents after packing a whole context (one layer).

    LeanK page, section 3.1 item 2 (K_cache for sink + local window, K_prun
    for the middle) and section 3.2 (no middle V for fully-pruned heads).

    k_bits, v_bits: uint16 [B, H, T, d] bf16 bit patterns of the context.
    kept_count: int [H]; kept_idx: int [H, d] (ascending, -1 padded).
    Returns a dict:
      ring_k, ring_v: uint16 [B, H, S + W, d] (unfilled slots are zero),
      slot_pos: int64 [S + W] position held by each slot (-1 = empty),
      k_prun: list over heads of uint16 [B, T_mid, c_h],
      v_mid: list over heads of uint16 [B, T_mid, d] or None (dead head).
    """
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    batch, n_heads, ctx_len, d = k_bits.shape
    sink, middle, local = regions(ctx_len, n_sink, window)
    n_slots = n_sink + window
    ring_k = np.zeros((batch, n_heads, n_slots, d), dtype=np.uint16)
    ring_v = np.zeros_like(ring_k)
    slot_pos = np.full(n_slots, -1, dtype=np.int64)
    for pos in list(sink) + list(local):
        slot = ring_slot(pos, n_sink, window)
        ring_k[:, :, slot, :] = k_bits[:, :, pos, :]
        ring_v[:, :, slot, :] = v_bits[:, :, pos, :]
        slot_pos[slot] = pos
    mid = np.asarray(list(middle), dtype=np.int64)
    k_prun, v_mid = [], []
    for head in range(n_heads):
        c = int(kept_count[head])
        chans = np.asarray(kept_idx[head][:c], dtype=np.int64)
        rows = k_bits[:, head][:, mid]  # [B, T_mid, d]
        k_prun.append(rows[:, :, chans].copy())
        v_mid.append(v_bits[:, head][:, mid].copy() if c > 0 else None)
    return {"ring_k": ring_k, "ring_v": ring_v, "slot_pos": slot_pos,
            "k_prun": k_prun, "v_mid": v_mid}


def _attend(shape, get_q, get_k, get_v, mask, n_sink, window, scale, pairs):
    """The attention definition over row accessors.

    shape = (B, Hq, H, T, d); get_q(b, j) -> float64 [d]; get_k(b, h, rows)
    and get_v(b, h, rows) -> float64 [len(rows), d].
    """
    batch, n_q_heads, n_heads, ctx_len, d = shape
    if ctx_len < 1:
        raise ValueError("empty context")
    group = n_q_heads // n_heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    sink, middle, local = regions(ctx_len, n_sink, window)
    full_rows = np.asarray(list(sink) + list(local), dtype=np.int64)
    mid_rows = np.asarray(list(middle), dtype=np.int64)

    if pairs is None:
        pairs = [(b, j) for b in range(batch) for j in range(n_q_heads)]
        out = np.zeros((batch, n_q_heads, d), dtype=np.float64)
        put = lambda b, j, val: out.__setitem__((b, j), val)
    else:
        # row n of the result answers pairs[n]; a pair listed twice is
        # computed once and written to every row that asks for it
        out = np.zeros((len(pairs), d), dtype=np.float64)
        index = {}
        for n, pair in enumerate(pairs):
            index.setdefault(tuple(pair), []).append(n)
        put = lambda b, j, val: out.__setitem__(index[(b, j)], val)

    by_kv = {}
    for b, j in dict.fromkeys(tuple(p) for p in pairs):
        by_kv.setdefault((b, j // group), []).append(j)
    for (b, h), heads in sorted(by_kv.items()):
        beta = np.asarray(mask[h], dtype=np.float64)
        live = bool(np.any(beta != 0))
        keys_full = get_k(b, h, full_rows)
        vals_full = get_v(b, h, full_rows)
        if live and mid_rows.size:
            keys_mid = get_k(b, h, mid_rows) * beta
            vals_mid = get_v(b, h, mid_rows)
            keys = np.concatenate([keys_full, keys_mid])
            vals = np.concatenate([vals_full, vals_mid])
        else:
            keys, vals = keys_full, vals_full
        for j in heads:
            qv = get_q(b, j)
            s = (keys @ qv) * scale
            w = np.exp(s - s.max())
            put(b, j, (w @ vals) / w.sum())
    return out


def decode(q_bits, k_bits, v_bits, mask, n_sink, window, scale=None, pairs=None):
    """Single-token decode attention over a channel-pruned cache (one layer).

    q_bits: uint16 [B, Hq, d]; k_bits, v_bits: uint16 [B, H, T, d] -- the
    full, unpruned context of T tokens; mask: uint8 [H, d] (beta of the
    LeanK page, section 2.2 stage 2).  Query head j reads KV head j // G.

    For query head j with KV head h (definition, float64):
      * sink and local-window tokens score q . k over all channels;
      * middle tokens of a head with kept channels score q . (beta_h * k);
      * middle tokens of a fully-pruned head are left out entirely;
      * out = sum_t softmax(scale * s)_t v_t over the included tokens,
        scale = 1/sqrt(d) by default (FastGen page, section 5.3).

    Returns float64 [B, Hq, d], or [len(pairs), d] for a list of (b, j).
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    batch, n_q_heads, d = q_bits.shape
    _, n_heads, ctx_len, _ = k_bits.shape
    return _attend((batch, n_q_heads, n_heads, ctx_len, d),
                   lambda b, j: bf16_bits_to_f64(q_bits[b, j]),
                   lambda b, h, rows: bf16_bits_to_f64(k_bits[b, h, rows]),
                   lambda b, h, rows: bf16_bits_to_f64(v_bits[b, h, rows]),
                   mask, n_sink, window, scale, pairs)



def decode_f64(q, k, v, mask, n_sink, window, scale=None, pairs=None):
    """decode() on values already widened to float64 (q [B, Hq, d], k, v
    [B, H, T, d]), the same definition step for step; lets a caller time the
    widening of the bf16 inputs apart from the attention itself."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    batch, n_q_heads, d = q.shape
    _, n_heads, ctx_len, _ = k.shape
    return _attend((batch, n_q_heads, n_heads, ctx_len, d),
                   lambda b, j: q[b, j],
                   lambda b, h, rows: k[b, h, rows],
                   lambda b, h, rows: v[b, h, rows],
                   mask, n_sink, window, scale, pairs)

# ---------------------------------------------------------------------------
# low-bit middle streams (LeanK page, section 4.2; white paper section 5.2.1)

QUANT_GROUP = 64  # middle rows per K quantization group


def quantize_asym(x, bits, axis):
    """Asymmetric uniform quantization of x along `axis` (one group per
    slice along the other axes).  Returns (codes uint8, scale float32, lo
    float32), scale and lo with the reduced axis kept (size 1).

    Decided in float32: lo = min, hi = max, scale = (hi - lo) / (2^bits - 1),
    code = rint((x - lo) / scale) clamped to [0, 2^bits - 1]; 0 when scale = 0.
    """
    x = np.asarray(x, dtype=np.float32)
    levels = np.float32(2 ** bits - 1)
    lo = x.min(axis=axis, keepdims=True)
    hi = x.max(axis=axis, keepdims=True)
    scale = (hi - lo) / levels
    with np.errstate(divide="ignore", invalid="ignore"):
        raw = np.rint((x - lo) / scale)
    codes = np.where(scale > 0, np.clip(raw, 0, levels), 0).astype(np.uint8)
    return codes, scale, lo


def dequantize(codes, scale, lo):
    """code * scale + lo, in float64 from the stored float32 scale and lo."""
    return (np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)
            + np.asarray(lo, dtype=np.float64))


def quantize_middle(k_prun_bits, v_mid_bits, bits, group=QUANT_GROUP):
    """Quantized middle of one (batch row, KV head) pair of a live head.

    k_prun_bits: uint16 [T_mid, c] (kept channels, bf16); v_mid_bits: uint16
    [T_mid, d].  Returns a dict:
      k_codes uint8 [n_full * group, c], k_scale / k_lo float32 [n_full, c]
        (per channel over each complete group of `group` rows),
      k_stage uint16 [T_mid - n_full * group, c] (rows of the incomplete
        group, bf16 as packed),
      v_codes uint8 [T_mid, d], v_scale / v_lo float32 [T_mid] (per token).
    """
    k_prun_bits = np.asarray(k_prun_bits, dtype=np.uint16)
    v_mid_bits = np.asarray(v_mid_bits, dtype=np.uint16)
    t_mid, c = k_prun_bits.shape
    n_full = t_mid // group
    k32 = bf16_bits_to_f64(k_prun_bits[:n_full * group]).astype(np.float32)
    k_codes, k_scale, k_lo = quantize_asym(k32.reshape(n_full, group, c), bits, axis=1)
    v32 = bf16_bits_to_f64(v_mid_bits).astype(np.float32)
    v_codes, v_scale, v_lo = quantize_asym(v32, bits, axis=1)
    return {"k_codes": k_codes.reshape(n_full * group, c),
            "k_scale": k_scale.reshape(n_full, c), "k_lo": k_lo.reshape(n_full, c),
            "k_stage": k_prun_bits[n_full * group:].copy(),
            "v_codes": v_codes, "v_scale": v_scale.reshape(t_mid), "v_lo": v_lo.reshape(t_mid)}


def pack_reference_q(k_bits, v_bits, kept_count, kept_idx, n_sink, window, bits,
                     group=QUANT_GROUP):
    """Expected contents of a cache with low-bit middle streams: the ring as
    in pack_reference, and for every (b, live h) the quantize_middle dict
    (None for a dead head)."""
    ref = pack_reference(k_bits, v_bits, kept_count, kept_idx, n_sink, window)
    batch = np.asarray(k_bits).shape[0]
    mid_q = []
    for head, kp in enumerate(ref["k_prun"]):
        if int(kept_count[head]) == 0:
            mid_q.append(None)
            continue
        mid_q.append([quantize_middle(kp[b], ref["v_mid"][head][b], bits, group)
                      for b in range(batch)])
    ref["mid_q"] = mid_q
    return ref


def decode_q(q_bits, k_bits, v_bits, mask, n_sink, window, bits, group=QUANT_GROUP,
             scale=None, pairs=None):
    """decode() with the middle of every live head read back from its
    low-bit streams: kept K channels of complete groups and every middle V
    row are replaced by their dequantized values; the rows of the incomplete
    K group, the sink and the window are exact."""
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    batch, n_q_heads, d = q_bits.shape
    _, n_heads, ctx_len, _ = k_bits.shape
    _, middle, _ = regions(ctx_len, n_sink, window)
    middle_pos = np.asarray(list(middle), dtype=np.int64)
    cache = {}

    def middle_of(b, h):
        if (b, h) not in cache:
            chans = np.flatnonzero(np.asarray(mask[h]))
            kq = quantize_middle(k_bits[b, h][middle_pos][:, chans], v_bits[b, h][middle_pos], bits, group)
            k = bf16_bits_to_f64(k_bits[b, h][middle_pos])
            n_q = kq["k_codes"].shape[0]
            k[:n_q, chans] = dequantize(kq["k_codes"].reshape(-1, group, chans.size),
                                        kq["k_scale"][:, None, :],
                                        kq["k_lo"][:, None, :]).reshape(n_q, chans.size)
            v = dequantize(kq["v_codes"], kq["v_scale"][:, None], kq["v_lo"][:, None])
            cache[(b, h)] = (k, v)
        return cache[(b, h)]

    def rows_of(bits_arr, which):
        def get(b, h, rows):
            out = bf16_bits_to_f64(bits_arr[b, h, rows])
            if middle_pos.size and np.any(mask[h]):
                at = rows - n_sink
                inside = (rows >= n_sink) & (at < middle_pos.size)
                if np.any(inside):
                    out[inside] = middle_of(b, h)[which][at[inside]]
            return out
        return get

    return _attend((batch, n_q_heads, n_heads, ctx_len, d),
                   lambda b, j: bf16_bits_to_f64(q_bits[b, j]),
                   rows_of(k_bits, 0), rows_of(v_bits, 1),
                   mask, n_sink, window, scale, pairs)


def kv_cache_bytes(n_layers, n_heads, head_dim, n_tokens, batch=1, bytes_per_elem=2):
    """Dense KV-cache size: 2 (K and V) x L x h x d x N per sequence.

    LeanK page, section 1.
    """
    return 2 * n_layers * n_heads * head_dim * n_tokens * batch * bytes_per_elem


def decode_traffic_bytes(batch, n_q_heads, n_kv_heads, head_dim, ctx_len,
                         n_sink, window, kept_count):
    """Bytes one pruned decode step must move for one layer.

    Reads q (bf16), the full-width sink+window keys and values of every head,
    the kept middle channels of K and the middle V of live heads (bf16), and
    writes the fp32 output.  Nothing else is counted.
    """
    sink, middle, local = regions(ctx_len, n_sink, window)
    n_full = len(sink) + len(local)
    n_mid = len(middle)
    kept = [int(c) for c in kept_count]
    live = sum(1 for c in kept if c > 0)
    total = batch * n_q_heads * head_dim * 2                      # q
    total += 2 * batch * n_kv_heads * n_full * head_dim * 2        # K, V full width
    total += batch * n_mid * sum(kept) * 2                         # kept K channels
    total += batch * live * n_mid * head_dim * 2                   # middle V, live heads
    total += batch * n_q_heads * head_dim * 4                      # out
    return total


def decode_traffic_bytes_q(batch, n_q_heads, n_kv_heads, head_dim, ctx_len, n_sink, window,
                           kept_count, bits, group=QUANT_GROUP):
    """decode_traffic_bytes with low-bit middle streams: per live head and
    batch row, the codes of the complete K groups (c * bits / 8 per row) and
    their float32 scale and minimum per channel and group, the bf16 rows of
    the incomplete group, and per middle row the V codes (d * bits / 8) and
    the row's float32 scale and minimum."""
    sink, middle, local = regions(ctx_len, n_sink, window)
    n_full_rows = len(sink) + len(local)
    n_mid = len(middle)
    n_groups = n_mid // group
    n_stage = n_mid - n_groups * group
    total = batch * n_q_heads * head_dim * 2                      # q
    total += 2 * batch * n_kv_heads * n_full_rows * head_dim * 2   # K, V full width
    for c in (int(x) for x in kept_count):
        if c == 0:
            continue
        k = n_groups * group * c * bits // 8 + n_groups * c * 8 + n_stage * c * 2
        v = n_mid * (head_dim * bits // 8 + 8)
        total += batch * (k + v)
    total += batch * n_q_heads * head_dim * 4                      # out
    return total


# ---------------------------------------------------------------------------
# alpha / mask analysis (LeanK page, section 6 and section 2.1)

def pair_retention(mask):
    """Fraction of (layer, head) rows keeping each rotate-half channel pair.

    LeanK page, section 6: lower pair indices (higher RoPE frequencies) are
    kept less often.  Pair i joins channels i and i + d/2; a head counts 1
    for a pair if both channels are kept, 1/2 if one is.
    mask: uint8 [L, H, d]  ->  float64 [d/2].
    """
    mask = np.asarray(mask)
    d = mask.shape[-1]
    half = d // 2
    rows = mask.reshape(-1, d).astype(np.float64)
    per_pair = (rows[:, :half] + rows[:, half:]) / 2.0
    return per_pair.mean(axis=0)


def head_hf_ratio(alpha, n_hf_pairs):
    """Share of each head's alpha mass on its n_hf_pairs highest-frequency pairs.

    LeanK page, section 6 (w_hf per head).  Reading: a pair's RoPE frequency
    falls with its index, so the highest-frequency pairs are the first
    n_hf_pairs; w_hf = sum of |alpha| over their channels / sum over all.
    alpha: float [L, H, d]  ->  float64 [L, H].
    """
    a = np.abs(np.asarray(alpha, dtype=np.float64))
    d = a.shape[-1]
    half = d // 2
    hf = a[..., :n_hf_pairs].sum(axis=-1) + a[..., half:half + n_hf_pairs].sum(axis=-1)
    total = a.sum(axis=-1)
    return np.where(total > 0, hf / np.where(total > 0, total, 1.0), 0.0)


def _average_ranks(x):
    """Ranks 1..n of x, ties given the mean of the ranks they span."""
    x = np.asarray(x, dtype=np.float64)
    order = sorted(range(x.size), key=lambda i: x[i])
    ranks = np.empty(x.size, dtype=np.float64)
    i = 0
    while i < x.size:
        j = i
        while j + 1 < x.size and x[order[j + 1]] == x[order[i]]:
            j += 1
        for k in range(i, j + 1):
            ranks[order[k]] = (i + j) / 2.0 + 1.0
        i = j + 1
    return ranks


def _pearson(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    dx = x - x.mean()
    dy = y - y.mean()
    den = np.sqrt((dx * dx).sum() * (dy * dy).sum())
    return float((dx * dy).sum() / den) if den > 0 else 0.0


def rank_correlation(a, b):
    """(Pearson of the values, Pearson of the average ranks) of two alphas.

    LeanK page, section 2.1: the channel-importance ranking is stable across
    tasks and lengths (a correlation near 0.98); comparing two alpha draws by
    the correlation of their rankings measures that stability.
    """
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return _pearson(a, b), _pearson(_average_ranks(a), _average_ranks(b))
