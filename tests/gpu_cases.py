"""Helpers for the GPU parity tests: build caches through the C ABI, read
their buffers back, and compare with the CPU oracle."""

import numpy as np
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits

# max |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise (bf16 inputs,
# float32 accumulation against a float64 oracle)
ATOL = 2e-3
RTOL = 1e-2


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), (
        f"{what}: max err {err.ravel()[worst]:.3e} > bound {bound.ravel()[worst]:.3e} "
        f"at {np.unravel_index(worst, err.shape)}")


def kept_from_mask(mask):
    """kept_count [H] and kept_idx [H, 128] (ascending, -1 padded) of a 0/1 mask [H, 128]."""
    mask = np.asarray(mask)
    n_heads, d = mask.shape
    kept_count = mask.sum(axis=1).astype(np.int32)
    kept_idx = np.full((n_heads, d), -1, dtype=np.int16)
    for h in range(n_heads):
        kept_idx[h, :kept_count[h]] = np.flatnonzero(mask[h])
    return kept_count, kept_idx


def mask_with_counts(rng, counts, d=128):
    mask = np.zeros((len(counts), d), dtype=np.uint8)
    for h, c in enumerate(counts):
        if c:
            mask[h, np.sort(rng.choice(d, size=c, replace=False))] = 1
    return mask


def make_cache(mask, batch, n_q, n_sink, window, max_ctx, device="cuda"):
    kept_count, kept_idx = kept_from_mask(mask)
    kept_dev = torch.from_numpy(kept_idx).to(device)
    return dac.LayerCache(kept_count.tolist(), kept_dev, batch, n_q, mask.shape[0], n_sink,
                          window, max_ctx, device=device)


def random_bf16(shape, gen, scale=1.0, device="cuda"):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return (x * scale).to(torch.bfloat16)


def _v_rows(rows):
    return (rows + 7) // 8 * 8


def _unblock_v(flat, rows):
    """Rows [rows, 128] of a V region stored in 8-row blocks
    (element (r, c) at ((r // 8) * 128 + c) * 8 + r % 8)."""
    blocks = flat.reshape(-1, 128, 8)          # [block][channel][row in block]
    return blocks.transpose(0, 2, 1).reshape(-1, 128)[:rows]


def read_pair(cache, b, h, n_mid=None, ring_only=False):
    """Host uint16 copies of one (batch row, KV head) pair's cache rows:
    ring K/V [slots, 128], K_prun [n_mid, kept] and V_mid [n_mid, 128] (None
    for a fully pruned head).  Slices on the GPU before copying."""
    d = cache.desc
    slots = d.n_sink + d.window
    mid_cap = d.mid_capacity
    n_mid = mid_cap if n_mid is None else n_mid
    base = ((b * d.n_kv_heads) + h) * slots * 128
    ring_k = bf16_bits(cache.k_sl[base: base + slots * 128]).reshape(slots, 128)
    vs = _v_rows(slots)
    vbase = ((b * d.n_kv_heads) + h) * vs * 128
    ring_v = _unblock_v(bf16_bits(cache.v_sl[vbase: vbase + vs * 128]), slots)
    c = d.kept_count[h]
    if c == 0 or ring_only:
        return ring_k, ring_v, None, None
    if d.page_rows:
        return ring_k, ring_v, *_read_paged_middle(cache, b, h, n_mid)
    ko = d.k_prun_off[h] + b * mid_cap * c
    k_prun = bf16_bits(cache.k_prun[ko: ko + n_mid * c]).reshape(n_mid, c)
    vm = _v_rows(mid_cap)
    vo = d.v_mid_off[h] + b * vm * 128
    nv = _v_rows(n_mid)
    v_mid = _unblock_v(bf16_bits(cache.v_mid[vo: vo + nv * 128]), n_mid)
    return ring_k, ring_v, k_prun, v_mid


def assert_cache_matches(cache, k_bits, v_bits, mask, pairs=None):
    """Bit-exact comparison of the cache with the oracle's packing of the
    full context k_bits/v_bits [B, H, T, d] (optionally for some (b, h) only:
    then k_bits/v_bits hold just those rows, in the order of `pairs`)."""
    d = cache.desc
    kept_count, kept_idx = kept_from_mask(mask)
    if pairs is None:
        pairs = [(b, h) for b in range(d.batch) for h in range(d.n_kv_heads)]
        rows = {(b, h): (b, h) for b, h in pairs}
    else:
        rows = {pair: (n, 0) for n, pair in enumerate(pairs)}
    for (b, h) in pairs:
        rb, rh = rows[(b, h)]
        one_k = k_bits[rb:rb + 1, rh:rh + 1]
        one_v = v_bits[rb:rb + 1, rh:rh + 1]
        ref = oracle.pack_reference(one_k, one_v, kept_count[h:h + 1], kept_idx[h:h + 1],
                                    d.n_sink, d.window)
        n_mid = ref["k_prun"][0].shape[1]
        ring_k, ring_v, k_prun, v_mid = read_pair(cache, b, h, n_mid)
        for slot, pos in enumerate(ref["slot_pos"]):
            if pos < 0:
                continue
            assert np.array_equal(ring_k[slot], ref["ring_k"][0, 0, slot]), (b, h, slot, pos)
            assert np.array_equal(ring_v[slot], ref["ring_v"][0, 0, slot]), (b, h, slot, pos)
        if kept_count[h] == 0:
            assert k_prun is None and ref["v_mid"][0] is None
            continue
        assert np.array_equal(k_prun, ref["k_prun"][0][0]), (b, h)
        assert np.array_equal(v_mid, ref["v_mid"][0][0]), (b, h)


def oracle_outputs(q, k, v, mask, n_sink, window, pairs=None):
    """Oracle decode for torch bf16 tensors (host copies of the same bits)."""
    return oracle.decode(bf16_bits(q), bf16_bits(k), bf16_bits(v), mask, n_sink, window,
                         pairs=pairs)


def _unpack_nibbles(b):
    """uint8 bytes -> codes, low nibble first."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.size * 2, dtype=np.uint8)
    out[0::2] = b & 0xF
    out[1::2] = b >> 4
    return out


def _read_paged_q(cache, b, h, t_mid):
    """read_pair_q for a paged low-bit middle: group g of the row in page
    block_table[b][g]."""
    d = cache.desc
    bits, c = d.quant_bits, d.kept_count[h]
    pool = cache.pool.view(torch.uint8).cpu().numpy()
    table = cache.block_table.cpu().numpy()
    n_full = t_mid // 64
    n_groups = -(-t_mid // 64)
    blk_bytes = 128 * 8 * bits // 8
    k_codes, kpar, v_codes, vpar = [], [], [], []
    for g in range(n_groups):
        base = int(table[b, g]) * d.page_bytes
        page = pool[base: base + d.page_bytes]
        if g < n_full:
            raw = page[d.k_q_off[h]: d.k_q_off[h] + 64 * c * bits // 8]
            k_codes.append((raw if bits == 8 else _unpack_nibbles(raw)).reshape(64, c))
            kp = page[4 * d.k_qp_off[h]: 4 * d.k_qp_off[h] + 8 * c].view(np.float32)
            kpar.append(kp.reshape(c, 2))
        vraw = page[d.v_q_off[h]: d.v_q_off[h] + 8 * blk_bytes]
        if bits == 8:
            codes = vraw.reshape(8, 128, 8)
        else:
            b4 = vraw.reshape(8, 128, 4)
            codes = np.concatenate([b4 & 0xF, b4 >> 4], axis=2)
        v_codes.append(codes.transpose(0, 2, 1).reshape(64, 128))
        vpar.append(page[4 * d.v_qp_off[h]: 4 * d.v_qp_off[h] + 512].view(np.float32).reshape(64, 2))
    st = cache.quant["k_stage"].cpu().numpy().view(np.uint16)
    s0 = d.k_stage_off[h] + b * 64 * c
    k_stage = st[s0: s0 + (t_mid - n_full * 64) * c].reshape(-1, c)
    k_codes = np.concatenate(k_codes) if k_codes else np.zeros((0, c), np.uint8)
    kpar = np.stack(kpar) if kpar else np.zeros((0, c, 2), np.float32)
    v_codes = np.concatenate(v_codes)[:t_mid] if v_codes else np.zeros((0, 128), np.uint8)
    vpar = np.concatenate(vpar)[:t_mid] if vpar else np.zeros((0, 2), np.float32)
    return {"k_codes": k_codes, "k_scale": kpar[..., 0], "k_lo": kpar[..., 1], "k_stage": k_stage,
            "v_codes": v_codes, "v_scale": vpar[:, 0], "v_lo": vpar[:, 1]}


def read_pair_q(cache, b, h, t_mid):
    """Host copies of one (batch row, live KV head) pair's low-bit middle
    for t_mid middle rows: a dict shaped like oracle.quantize_middle."""
    d = cache.desc
    if d.page_rows:
        return _read_paged_q(cache, b, h, t_mid)
    bits, c = d.quant_bits, d.kept_count[h]
    g_rows = -(-d.mid_capacity // 64) * 64
    n_full = t_mid // 64
    q = {name: t.cpu().numpy() for name, t in cache.quant.items()}
    k0 = d.k_q_off[h] + b * g_rows * c * bits // 8
    raw = q["k_q"][k0: k0 + n_full * 64 * c * bits // 8]
    k_codes = (raw if bits == 8 else _unpack_nibbles(raw)).reshape(n_full * 64, c)
    kp = q["k_qp"].view(np.float32)
    p0 = d.k_qp_off[h] + b * (g_rows // 64) * c * 2
    kpar = kp[p0: p0 + n_full * c * 2].reshape(n_full, c, 2)
    st = q["k_stage"].view(np.uint16)
    s0 = d.k_stage_off[h] + b * 64 * c
    k_stage = st[s0: s0 + (t_mid - n_full * 64) * c].reshape(-1, c)
    vrows = _v_rows(d.mid_capacity)
    blk_bytes = 128 * 8 * bits // 8
    v0 = d.v_q_off[h] + b * (vrows // 8) * blk_bytes
    nb = -(-t_mid // 8)
    vraw = q["v_q"][v0: v0 + nb * blk_bytes]
    if bits == 8:
        codes = vraw.reshape(nb, 128, 8)
    else:  # byte k of a channel's 4 bytes: row k (low nibble), row k + 4 (high nibble)
        b4 = vraw.reshape(nb, 128, 4)
        codes = np.concatenate([b4 & 0xF, b4 >> 4], axis=2)
    v_codes = codes.transpose(0, 2, 1).reshape(-1, 128)[:t_mid]
    vp = q["v_qp"].view(np.float32)
    q0 = d.v_qp_off[h] + b * d.mid_capacity * 2
    vpar = vp[q0: q0 + t_mid * 2].reshape(t_mid, 2)
    return {"k_codes": k_codes, "k_scale": kpar[..., 0], "k_lo": kpar[..., 1], "k_stage": k_stage,
            "v_codes": v_codes, "v_scale": vpar[:, 0], "v_lo": vpar[:, 1]}


def assert_quant_cache_matches(cache, k_bits, v_bits, mask, pairs=None, rows=None):
    """Bit-exact comparison of a low-bit cache (ring and middle streams) with
    the oracle's packing of the full context k_bits/v_bits [B, H, T, d].
    rows: the cache rows that k_bits' batch entries belong to (default: the
    same index), so one row of a ragged batch can be checked on its own."""
    d = cache.desc
    kept_count, kept_idx = kept_from_mask(mask)
    rows = list(range(k_bits.shape[0])) if rows is None else list(rows)
    if pairs is None:
        pairs = [(rb, h) for rb in range(len(rows)) for h in range(d.n_kv_heads)]
    ref = oracle.pack_reference_q(k_bits, v_bits, kept_count, kept_idx, d.n_sink, d.window,
                                  d.quant_bits)
    for (rb, h) in pairs:
        b = rows[rb]
        ring_k, ring_v, _, _ = read_pair(cache, b, h, ring_only=True)
        for slot, pos in enumerate(ref["slot_pos"]):
            if pos < 0:
                continue
            assert np.array_equal(ring_k[slot], ref["ring_k"][rb, h, slot]), (b, h, slot)
            assert np.array_equal(ring_v[slot], ref["ring_v"][rb, h, slot]), (b, h, slot)
        if kept_count[h] == 0:
            continue
        want = ref["mid_q"][h][rb]
        got = read_pair_q(cache, b, h, want["v_codes"].shape[0])
        for key in ("k_codes", "k_stage", "v_codes"):
            assert np.array_equal(got[key], want[key]), (b, h, key)
        for key in ("k_scale", "k_lo", "v_scale", "v_lo"):
            assert np.array_equal(got[key].view(np.uint32), want[key].view(np.uint32)), (b, h, key)


def _read_paged_middle(cache, b, h, n_mid):
    """K_prun [n_mid, kept] and V_mid [n_mid, 128] of a paged cache, gathered
    page by page through the block table."""
    d = cache.desc
    c = d.kept_count[h]
    pe = d.page_bytes // 2
    pool = bf16_bits(cache.pool)
    table = cache.block_table.cpu().numpy()
    k_rows, v_rows = [], []
    for p0 in range(0, n_mid, 64):
        page = int(table[b, p0 // 64])
        base = page * pe
        n = min(64, n_mid - p0)
        k_rows.append(pool[base + d.k_prun_off[h]: base + d.k_prun_off[h] + 64 * c].reshape(64, c)[:n])
        v_rows.append(_unblock_v(pool[base + d.v_mid_off[h]: base + d.v_mid_off[h] + 64 * 128], 64)[:n])
    if not k_rows:
        return np.zeros((0, c), np.uint16), np.zeros((0, 128), np.uint16)
    return np.concatenate(k_rows), np.concatenate(v_rows)


def shuffled_block_table(rng, batch, pages_per_row, n_pages, device="cuda"):
    """A block table giving every (batch row, page) a distinct pool page in
    random order."""
    pick = rng.permutation(n_pages)[:batch * pages_per_row]
    return torch.from_numpy(pick.astype(np.int32).reshape(batch, pages_per_row)).to(device)


# cache kinds of the seeded random layers
KINDS = ["bf16", "paged", "q4", "q8", "paged_q4"]


def build_kind(kind, mask, batch, n_q, n_sink, window, max_ctx, seed):
    """A cache of one of KINDS for `mask`: bf16, paged bf16 (64-row pages
    through a shuffled block table), 4- or 8-bit middles, paged 4-bit.
    Returns (cache, bits)."""
    kept_count, kept_idx = kept_from_mask(mask)
    kw = {}
    if kind.startswith("paged"):
        mid_cap = max(0, max_ctx - n_sink - window)
        ppr = -(-mid_cap // 64)
        n_pages = batch * ppr + 3
        kw = dict(n_pages=n_pages,
                  block_table=shuffled_block_table(np.random.default_rng(seed), batch, ppr, n_pages))
    bits = {"q4": 4, "q8": 8, "paged_q4": 4}.get(kind, 0)
    if bits:
        kw["quant_bits"] = bits
    cache = dac.LayerCache(kept_count.tolist(), torch.from_numpy(kept_idx).to("cuda"), batch, n_q,
                           mask.shape[0], n_sink, window, max_ctx, device="cuda", **kw)
    return cache, bits
