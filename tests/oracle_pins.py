"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an oracle module and raises AssertionError when
the module disagrees with:

* the stage-2 procedure of the LeanK page ("大型语言模型KV缓存优化与LeanK剪枝技术解析",
  section 2.2) run with library routines (numpy's linear-interpolation
  percentile and torch.topk) on tie-free inputs;
* closed forms and invariants of that procedure;
* brute-force enumeration of every kept-channel subset on tiny heads;
* torch's scaled_dot_product_attention in float64 (the textbook softmax
  attention with scale 1/sqrt(d), FastGen page section 5.3) on inputs where
  the pruned method reduces to it: channel-masked K on the middle tokens and
  a boolean mask that hides the middle tokens of fully-pruned heads;
* closed forms of softmax attention (uniform weights, constant values,
  one-token contexts, a single dominant key);
* a pure-Python attention loop on tiny inputs;
* the KV-cache sizes the pages work out (tests/golden/kv_cache_sizes.json);
* for the low-bit middle streams: values already on a quantization grid
  come back exactly, every value lands on its nearest level (brute force
  over all levels), values half-way between two levels take the even code,
  each group's minimum and maximum land on the end levels, every (batch row,
  live head) of a low-bit pack gives back its own middle exactly on
  grid-exact inputs, attention over grid-exact caches equals the unquantized
  definition, and the byte count equals the size of the packed arrays.

The same functions run against deliberately broken copies of the oracle in
test_oracle_mutants.py, which shows that each plausible slip is caught.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers (test-side formulations, written independently of the oracle)

def _f32_to_bf16_bits(x):
    """Round float values to bf16 bit patterns (round to nearest even) via torch."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(torch.float64)


def _is_full_width(t, ctx_len, n_sink, window):
    """Sink tokens and the last `window` tokens keep every K channel."""
    return t < n_sink or t >= ctx_len - window


def _tie_free_alpha(rng, shape):
    # distinct float32 values with overwhelming probability; re-draw if not
    while True:
        a = rng.random(shape).astype(np.float32) * 3.0
        if np.unique(a).size == a.size:
            return a


def _page_mask(alpha, prune_pct, align):
    """Stage 2 of LeanK section 2.2 with library routines (prune_pct = prune ratio)."""
    values = alpha.astype(np.float64)
    threshold = np.percentile(values.ravel(), prune_pct)
    keep = values >= threshold
    mask = np.zeros(alpha.shape, dtype=np.uint8)
    for layer in range(alpha.shape[0]):
        for head in range(alpha.shape[1]):
            n_keep = int(keep[layer, head].sum())
            n_keep = (n_keep // align) * align
            top = torch.topk(torch.from_numpy(values[layer, head]), k=n_keep).indices
            mask[layer, head, top.numpy()] = 1
    return mask


def _check_mask_outputs(alpha, mask, kept_count, kept_idx, align):
    assert mask.dtype == np.uint8 and kept_count.dtype == np.int32 and kept_idx.dtype == np.int16
    n_layers, n_heads, d = alpha.shape
    assert mask.shape == (n_layers, n_heads, d)
    assert kept_count.shape == (n_layers, n_heads) and kept_idx.shape == (n_layers, n_heads, d)
    assert np.all(kept_count % align == 0)
    for layer in range(n_layers):
        for head in range(n_heads):
            c = int(kept_count[layer, head])
            on = np.flatnonzero(mask[layer, head])
            assert on.size == c
            assert np.array_equal(kept_idx[layer, head, :c].astype(np.int64), on)
            assert np.all(kept_idx[layer, head, c:] == -1)


def _sdpa(q, k, v, attn_mask=None):
    """torch SDPA in float64 on CPU; q [B, Hq, d], k/v [B, Hq, T, d]."""
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, :, None, :], k, v, attn_mask=attn_mask)
    return out[:, :, 0, :].numpy()


def _random_case(rng, batch, n_q, n_kv, d, ctx_len, scale_k=1.0):
    q = _f32_to_bf16_bits(rng.standard_normal((batch, n_q, d)))
    k = _f32_to_bf16_bits(rng.standard_normal((batch, n_kv, ctx_len, d)) * scale_k)
    v = _f32_to_bf16_bits(rng.standard_normal((batch, n_kv, ctx_len, d)))
    return q, k, v


def _random_mask(rng, n_kv, d, align, dead_heads=()):
    mask = np.zeros((n_kv, d), dtype=np.uint8)
    for h in range(n_kv):
        if h in dead_heads:
            continue
        c = int(rng.integers(1, d // align + 1)) * align
        mask[h, rng.choice(d, size=c, replace=False)] = 1
    return mask


def _reference_masked(q, k, v, mask, n_sink, window):
    """Pruned decode through torch SDPA: masked K on middle tokens, dead middles hidden."""
    batch, n_q, d = q.shape
    n_kv, ctx_len = k.shape[1], k.shape[2]
    group = n_q // n_kv
    qf, kf, vf = _bits_to_f64(q), _bits_to_f64(k), _bits_to_f64(v)
    beta = torch.from_numpy(mask.astype(np.float64))
    middle = torch.tensor([not _is_full_width(t, ctx_len, n_sink, window) for t in range(ctx_len)])
    k_masked = kf.clone()
    k_masked[:, :, middle, :] *= beta[None, :, None, :]
    k_rep = k_masked.repeat_interleave(group, dim=1)
    v_rep = vf.repeat_interleave(group, dim=1)
    dead = torch.from_numpy(mask.sum(axis=1) == 0).repeat_interleave(group)
    allowed = torch.ones(batch, n_q, 1, ctx_len, dtype=torch.bool)
    allowed[:, dead.nonzero().flatten(), 0, :] = ~middle
    return _sdpa(qf, k_rep, v_rep, attn_mask=allowed)


# ----------------------------------------------------------------------------
# mask pins (LeanK page, section 2.2 stage 2)

def pin_mask_page_procedure(O):
    rng = np.random.default_rng(7)
    shapes = [(1, 2, 8), (2, 3, 16), (1, 8, 128), (3, 4, 64), (2, 8, 128)]
    for shape in shapes:
        d = shape[2]
        aligns = [a for a in (1, 2, 4, 8, 16, 32, 64) if d % a == 0]
        for p in (0, 1, 10, 33, 50, 70, 80, 97, 99, 100):
            alpha = _tie_free_alpha(rng, shape)
            for align in aligns:
                mask, kept_count, kept_idx = O.build_mask(alpha, p, align)
                assert np.array_equal(mask, _page_mask(alpha, p, align)), (shape, p, align)
                _check_mask_outputs(alpha, mask, kept_count, kept_idx, align)


def pin_mask_closed_forms(O):
    rng = np.random.default_rng(11)
    for shape in [(1, 2, 8), (2, 4, 32), (1, 8, 128)]:
        n = int(np.prod(shape))
        d = shape[2]
        alpha = _tie_free_alpha(rng, shape)
        # nothing pruned: every head keeps every channel
        _, kept_count, _ = O.build_mask(alpha, 0, 2)
        assert np.all(kept_count == d)
        # everything pruned: at most the global maximum survives the threshold
        _, kept_count, _ = O.build_mask(alpha, 100, 2)
        assert np.all(kept_count == 0)
        mask, kept_count, _ = O.build_mask(alpha, 100, 1)
        assert kept_count.sum() == 1
        assert mask.ravel()[np.argmax(alpha.ravel())] == 1
        # align 1: the kept total is N minus the percentile rank
        for p in (0, 5, 37, 50, 70, 93, 100):
            _, kept_count, _ = O.build_mask(alpha, p, 1)
            rank = math.ceil(Fraction((n - 1) * p, 100))
            assert kept_count.sum() == n - rank, (shape, p)


def pin_mask_invariants(O):
    rng = np.random.default_rng(13)
    cases = []
    for _ in range(6):
        cases.append(rng.integers(0, 4, size=(2, 4, 16)).astype(np.float32))  # many ties
    cases.append(np.where(rng.random((2, 3, 32)) < 0.3, np.float32(0.0), np.float32(-0.0)))
    mixed = rng.standard_normal((3, 4, 32)).astype(np.float32)
    mixed[0, 0, 3] = np.inf
    mixed[1, 2, 5] = -np.inf
    cases.append(mixed)
    for alpha in cases:
        d = alpha.shape[2]
        for p in (0, 20, 50, 75, 100):
            for align in (1, 2, 4, 8):
                if d % align:
                    continue
                mask, kept_count, kept_idx = O.build_mask(alpha, p, align)
                _check_mask_outputs(alpha, mask, kept_count, kept_idx, align)
                # numpy's "higher" order statistic selects the same channels as
                # linear interpolation on finite data and stays defined at +-inf
                threshold = np.percentile(alpha.astype(np.float64).ravel(), p, method="higher")
                for layer in range(alpha.shape[0]):
                    for head in range(alpha.shape[1]):
                        a = alpha[layer, head].astype(np.float64)
                        cnt = int((a >= threshold).sum())
                        c = int(kept_count[layer, head])
                        assert cnt - align < c <= cnt
                        kept = mask[layer, head].astype(bool)
                        if kept.any() and (~kept).any():
                            assert a[kept].min() >= a[~kept].max()
                            for i in np.flatnonzero(kept):
                                for j in np.flatnonzero(~kept):
                                    if a[i] == a[j]:
                                        assert i < j


def pin_mask_bruteforce(O):
    rng = np.random.default_rng(17)
    d = 8
    alphas = [rng.integers(0, 4, size=(1, 2, d)).astype(np.float32) for _ in range(4)]
    alphas += [_tie_free_alpha(rng, (1, 2, d)) for _ in range(2)]
    for alpha in alphas:
        values = alpha.astype(np.float64)
        for p in range(0, 101, 10):
            threshold = np.percentile(values.ravel(), p)
            for align in (1, 2, 4, 8):
                mask, kept_count, _ = O.build_mask(alpha, p, align)
                for head in range(2):
                    a = values[0, head]
                    c = (int((a >= threshold).sum()) // align) * align
                    valid = []
                    for subset in itertools.combinations(range(d), c):
                        inside = set(subset)
                        ok = all(a[i] > a[j] or (a[i] == a[j] and i < j)
                                 for i in inside for j in range(d) if j not in inside)
                        if ok:
                            valid.append(subset)
                    assert len(valid) == 1
                    expect = np.zeros(d, dtype=np.uint8)
                    expect[list(valid[0])] = 1
                    assert np.array_equal(mask[0, head], expect), (alpha, p, align, head)
                    assert kept_count[0, head] == c


# ----------------------------------------------------------------------------
# pack pins (LeanK page, section 3.1 item 2 and section 3.2)

def pin_pack_layout(O):
    rng = np.random.default_rng(19)
    batch, n_kv, d = 2, 3, 16
    for n_sink, window in ((2, 5), (4, 8), (0, 6), (3, 1)):
        for ctx_len in sorted({1, max(1, n_sink - 1), max(1, n_sink), n_sink + window - 1,
                               n_sink + window, n_sink + window + 1, n_sink + 3 * window + 5}):
            pos_code = np.broadcast_to(np.arange(ctx_len, dtype=np.uint16)[None, None, :, None],
                                       (batch, n_kv, ctx_len, d)).copy()
            chan_code = np.broadcast_to(np.arange(d, dtype=np.uint16) + 1000,
                                        (batch, n_kv, ctx_len, d)).copy()
            mask = _random_mask(rng, n_kv, d, 4, dead_heads=(1,))
            kept_count = mask.sum(axis=1).astype(np.int32)
            kept_idx = np.full((n_kv, d), -1, dtype=np.int16)
            for h in range(n_kv):
                kept_idx[h, :kept_count[h]] = np.flatnonzero(mask[h])
            full = [t for t in range(ctx_len) if _is_full_width(t, ctx_len, n_sink, window)]
            middle = [t for t in range(ctx_len) if not _is_full_width(t, ctx_len, n_sink, window)]

            by_pos = O.pack_reference(pos_code, pos_code + 7, kept_count, kept_idx, n_sink, window)
            by_chan = O.pack_reference(chan_code, chan_code, kept_count, kept_idx, n_sink, window)
            slot_pos = by_pos["slot_pos"]
            held = sorted(int(p) for p in slot_pos if p >= 0)
            assert held == full, (n_sink, window, ctx_len)
            for slot, pos in enumerate(slot_pos):
                if pos < 0:
                    continue
                if pos < n_sink:
                    assert slot == pos
                else:
                    assert n_sink <= slot < n_sink + window
                    assert (slot - n_sink) % window == (pos - n_sink) % window
                assert np.all(by_pos["ring_k"][:, :, slot, :] == pos)
                assert np.all(by_pos["ring_v"][:, :, slot, :] == pos + 7)
                assert np.all(by_chan["ring_k"][:, :, slot, :] == np.arange(d) + 1000)
            for h in range(n_kv):
                c = int(kept_count[h])
                kp = by_pos["k_prun"][h]
                assert kp.shape == (batch, len(middle), c)
                assert np.all(kp == np.asarray(middle, dtype=np.uint16)[None, :, None])
                chans = np.flatnonzero(mask[h]) + 1000
                assert np.all(by_chan["k_prun"][h] == chans[None, None, :].astype(np.uint16))
                if c == 0:
                    assert by_pos["v_mid"][h] is None
                else:
                    vm = by_pos["v_mid"][h]
                    assert vm.shape == (batch, len(middle), d)
                    assert np.all(vm == (np.asarray(middle) + 7).astype(np.uint16)[None, :, None])


def pin_pack_round_trip(O):
    """Unpacking the cache gives full K on full-width rows and beta-masked K in the middle."""
    rng = np.random.default_rng(23)
    batch, n_kv, d, n_sink, window = 2, 3, 32, 3, 7
    for ctx_len in (5, 10, 11, 40):
        _, k, v = _random_case(rng, batch, n_kv, n_kv, d, ctx_len)
        mask = _random_mask(rng, n_kv, d, 8, dead_heads=(2,))
        kept_count = mask.sum(axis=1).astype(np.int32)
        kept_idx = np.full((n_kv, d), -1, dtype=np.int16)
        for h in range(n_kv):
            kept_idx[h, :kept_count[h]] = np.flatnonzero(mask[h])
        packed = O.pack_reference(k, v, kept_count, kept_idx, n_sink, window)
        dense = np.zeros_like(k)
        for slot, pos in enumerate(packed["slot_pos"]):
            if pos >= 0:
                dense[:, :, pos, :] = packed["ring_k"][:, :, slot, :]
        middle = [t for t in range(ctx_len) if not _is_full_width(t, ctx_len, n_sink, window)]
        for h in range(n_kv):
            for r, t in enumerate(middle):
                dense[:, h, t, kept_idx[h, :kept_count[h]]] = packed["k_prun"][h][:, r, :]
        expect = k.copy()
        for t in middle:
            expect[:, :, t, :] = np.where(mask[None, :, :] == 1, k[:, :, t, :], 0)
        assert np.array_equal(dense, expect)


# ----------------------------------------------------------------------------
# decode pins

def pin_decode_dense_matches_sdpa(O):
    rng = np.random.default_rng(29)
    for batch, n_q, n_kv, d in ((2, 4, 2, 16), (1, 7, 1, 32), (1, 4, 4, 128), (2, 8, 2, 64)):
        for n_sink, window, ctx_len in ((2, 4, 1), (2, 4, 5), (2, 4, 6), (2, 4, 7), (3, 5, 30), (0, 4, 9)):
            q, k, v = _random_case(rng, batch, n_q, n_kv, d, ctx_len)
            mask = np.ones((n_kv, d), dtype=np.uint8)
            got = O.decode(q, k, v, mask, n_sink, window)
            group = n_q // n_kv
            expect = _sdpa(_bits_to_f64(q), _bits_to_f64(k).repeat_interleave(group, 1),
                           _bits_to_f64(v).repeat_interleave(group, 1))
            np.testing.assert_allclose(got, expect, rtol=1e-10, atol=1e-12)


def pin_decode_masked_matches_sdpa(O):
    rng = np.random.default_rng(31)
    for batch, n_q, n_kv, d, align in ((2, 4, 2, 32, 8), (1, 8, 4, 128, 32), (2, 6, 3, 64, 16)):
        for n_sink, window, ctx_len in ((2, 4, 7), (3, 5, 30), (0, 6, 25), (4, 8, 12), (1, 1, 9)):
            q, k, v = _random_case(rng, batch, n_q, n_kv, d, ctx_len, scale_k=2.0)
            mask = _random_mask(rng, n_kv, d, align, dead_heads=(n_kv - 1,))
            got = O.decode(q, k, v, mask, n_sink, window)
            expect = _reference_masked(q, k, v, mask, n_sink, window)
            np.testing.assert_allclose(got, expect, rtol=1e-10, atol=1e-12)
            # the entry point on values already widened to float64
            wide = O.decode_f64(_bits_to_f64(q).numpy(), _bits_to_f64(k).numpy(),
                                _bits_to_f64(v).numpy(), mask, n_sink, window)
            np.testing.assert_allclose(wide, expect, rtol=1e-10, atol=1e-12)
            # sampled-pairs entry point returns the same rows, in the order
            # asked, a pair asked twice in both rows
            pairs = [(batch - 1, n_q - 1), (0, 0), (batch - 1, n_q - 1), (0, 0)]
            sampled = O.decode(q, k, v, mask, n_sink, window, pairs=pairs)
            for n, (b, j) in enumerate(pairs):
                np.testing.assert_allclose(sampled[n], expect[b, j], rtol=1e-10, atol=1e-12)


def pin_decode_closed_forms(O):
    rng = np.random.default_rng(37)
    batch, n_q, n_kv, d, n_sink, window = 1, 4, 2, 16, 2, 3
    for ctx_len in (1, 2, 5, 6, 12):
        _, k, v = _random_case(rng, batch, n_q, n_kv, d, ctx_len)
        mask = np.zeros((n_kv, d), dtype=np.uint8)
        mask[0, :4] = 1                   # head 0 keeps 4 channels, head 1 is dead
        zero_q = np.zeros((batch, n_q, d), dtype=np.uint16)
        got = O.decode(zero_q, k, v, mask, n_sink, window)
        vf = _bits_to_f64(v).numpy()
        for j in range(n_q):
            h = j // (n_q // n_kv)
            rows = [t for t in range(ctx_len)
                    if _is_full_width(t, ctx_len, n_sink, window) or h == 0]
            np.testing.assert_allclose(got[0, j], vf[0, h, rows].mean(axis=0), rtol=1e-12, atol=1e-14)
        # constant value rows: the output is that row whatever the scores
        q, k2, _ = _random_case(rng, batch, n_q, n_kv, d, ctx_len)
        row = _f32_to_bf16_bits(rng.standard_normal(d))
        v_const = np.broadcast_to(row, v.shape).copy()
        got = O.decode(q, k2, v_const, mask, n_sink, window)
        np.testing.assert_allclose(got, np.broadcast_to(_bits_to_f64(row).numpy(), got.shape),
                                   rtol=1e-12, atol=1e-14)
    # a single token: the output is its value row
    q, k, v = _random_case(rng, 2, 4, 2, 16, 1)
    got = O.decode(q, k, v, np.zeros((2, 16), dtype=np.uint8), 0, 4)
    vf = _bits_to_f64(v).numpy()
    for j in range(4):
        np.testing.assert_allclose(got[:, j], vf[:, j // 2, 0], rtol=0, atol=0)
    # contexts that fit in sink + window do not depend on the mask
    for ctx_len in (3, 6, 7):
        q, k, v = _random_case(rng, 1, 4, 2, 16, ctx_len)
        a = O.decode(q, k, v, np.ones((2, 16), dtype=np.uint8), 3, 4)
        b = O.decode(q, k, v, np.zeros((2, 16), dtype=np.uint8), 3, 4)
        np.testing.assert_array_equal(a, b)
    # one dominant middle key: it wins only through a kept channel
    n_sink, window, ctx_len, star = 2, 3, 10, 4
    k = np.zeros((1, 1, ctx_len, d), dtype=np.uint16)
    k[0, 0, star, 5] = _f32_to_bf16_bits(np.float32(200.0))
    k[0, 0, ctx_len - 1, 9] = _f32_to_bf16_bits(np.float32(200.0))   # a window key
    v = _f32_to_bf16_bits(rng.standard_normal((1, 1, ctx_len, d)))
    vf = _bits_to_f64(v).numpy()[0, 0]
    q = np.zeros((1, 1, d), dtype=np.uint16)
    q[0, 0, 5] = _f32_to_bf16_bits(np.float32(1.0))
    kept = np.zeros((1, d), dtype=np.uint8)
    kept[0, :8] = 1                                     # channel 5 kept
    got = O.decode(q, k, v, kept, n_sink, window)[0, 0]
    np.testing.assert_allclose(got, vf[star], rtol=1e-12, atol=1e-12)
    pruned = np.zeros((1, d), dtype=np.uint8)
    pruned[0, 8:] = 1                                   # channel 5 pruned
    got = O.decode(q, k, v, pruned, n_sink, window)[0, 0]
    np.testing.assert_allclose(got, vf.mean(axis=0), rtol=1e-12, atol=1e-14)
    # the window key is full width even on a channel the head prunes
    q2 = np.zeros((1, 1, d), dtype=np.uint16)
    q2[0, 0, 9] = _f32_to_bf16_bits(np.float32(1.0))
    got = O.decode(q2, k, v, kept, n_sink, window)[0, 0]
    np.testing.assert_allclose(got, vf[ctx_len - 1], rtol=1e-12, atol=1e-12)


def pin_decode_bruteforce(O):
    """Pure-Python softmax attention over every 32-channel block pattern of each head."""
    rng = np.random.default_rng(41)
    batch, n_q, n_kv, d, n_sink, window, ctx_len = 1, 4, 2, 128, 2, 5, 14
    q, k, v = _random_case(rng, batch, n_q, n_kv, d, ctx_len)
    qf = _bits_to_f64(q).tolist()
    kf = _bits_to_f64(k).tolist()
    vf = _bits_to_f64(v).tolist()
    scale = 1.0 / math.sqrt(d)
    patterns = list(itertools.product((0, 1), repeat=4))
    combos = [(pa, (1, 0, 1, 0)) for pa in patterns] + [((0, 1, 1, 0), pb) for pb in patterns]
    for pa, pb in combos:
        mask = np.zeros((n_kv, d), dtype=np.uint8)
        for h, pat in enumerate((pa, pb)):
            for blk, on in enumerate(pat):
                if on:
                    mask[h, 32 * blk: 32 * blk + 32] = 1
        got = O.decode(q, k, v, mask, n_sink, window)
        for j in range(n_q):
            h = j // 2
            live = any(mask[h])
            scores, rows = [], []
            for t in range(ctx_len):
                full = t < n_sink or t >= ctx_len - window
                if not full and not live:
                    continue
                s = 0.0
                for x in range(d):
                    if full or mask[h, x]:
                        s += qf[0][j][x] * kf[0][h][t][x]
                scores.append(s * scale)
                rows.append(t)
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            total = sum(w)
            for x in range(0, d, 17):
                ref = sum(wi * vf[0][h][t][x] for wi, t in zip(w, rows)) / total
                assert abs(got[0, j, x] - ref) <= 1e-12 * max(1.0, abs(ref)), (pa, pb, j, x)


# ----------------------------------------------------------------------------
# byte accounting

def pin_cache_bytes(O):
    with open(os.path.join(GOLDEN, "kv_cache_sizes.json")) as fh:
        cases = json.load(fh)["cases"]
    for case in cases:
        got = O.kv_cache_bytes(case["layers"], case["kv_heads"], case["head_dim"],
                               case["tokens"], case["batch"], case["bytes_per_elem"])
        if "exact_bytes" in case:
            assert got == case["exact_bytes"], case["source"]
        lo, hi = case["approx_gib_range"]
        assert lo <= got / 2 ** 30 <= hi, case["source"]
        if "per_token_per_head_per_layer_bytes" in case:
            per = O.kv_cache_bytes(1, 1, case["head_dim"], 1, 1, case["bytes_per_elem"])
            assert per == case["per_token_per_head_per_layer_bytes"]


def pin_traffic_bytes(O):
    rng = np.random.default_rng(43)
    for batch, n_q, n_kv, d, n_sink, window, ctx_len in (
            (64, 32, 8, 128, 64, 512, 4096), (2, 4, 2, 16, 2, 3, 1), (3, 6, 3, 32, 4, 4, 20)):
        n_full = sum(_is_full_width(t, ctx_len, n_sink, window) for t in range(ctx_len))
        n_mid = ctx_len - n_full
        io = batch * n_q * d * 2 + batch * n_q * d * 4
        dense = O.decode_traffic_bytes(batch, n_q, n_kv, d, ctx_len, n_sink, window, [d] * n_kv)
        assert dense == io + 2 * batch * n_kv * ctx_len * d * 2
        dead = O.decode_traffic_bytes(batch, n_q, n_kv, d, ctx_len, n_sink, window, [0] * n_kv)
        assert dead == io + 2 * batch * n_kv * n_full * d * 2
        kept = [int(x) for x in rng.integers(0, d // 8 + 1, size=n_kv) * 8]
        mixed = O.decode_traffic_bytes(batch, n_q, n_kv, d, ctx_len, n_sink, window, kept)
        expect = dead + sum(batch * n_mid * (c * 2 + (d * 2 if c else 0)) for c in kept)
        assert mixed == expect


# ----------------------------------------------------------------------------
# alpha / mask analysis

def pin_analysis(O):
    from scipy import stats

    rng = np.random.default_rng(47)
    # retention: closed forms and a hand count
    d = 16
    mask = np.zeros((2, 3, d), dtype=np.uint8)
    mask[0, 0, [0, 8]] = 1          # pair 0 fully kept by one head
    mask[1, 2, 3] = 1               # half of pair 3 in one head
    ret = O.pair_retention(mask)
    assert ret.shape == (8,)
    assert ret[0] == 1.0 / 6 and ret[3] == 0.5 / 6 and ret[[1, 2, 4, 5, 6, 7]].sum() == 0
    assert np.all(O.pair_retention(np.ones((2, 2, d), dtype=np.uint8)) == 1.0)
    # w_hf: uniform alpha gives n_hf / (d/2); mass only on the first pair gives 1
    a = np.ones((2, 2, 32))
    assert np.allclose(O.head_hf_ratio(a, 4), 4 / 16)
    b = np.zeros((1, 1, 32))
    b[0, 0, [0, 16]] = [3.0, 1.0]
    assert O.head_hf_ratio(b, 1)[0, 0] == 1.0 and O.head_hf_ratio(b, 0)[0, 0] == 0.0
    # correlations against scipy, with and without ties
    for x, y in ((rng.standard_normal(200), rng.standard_normal(200)),
                 (rng.integers(0, 5, 300).astype(float), rng.integers(0, 5, 300).astype(float))):
        y2 = x + 0.3 * y
        pear, spear = O.rank_correlation(x, y2)
        assert abs(pear - stats.pearsonr(x, y2)[0]) < 1e-12
        assert abs(spear - stats.spearmanr(x, y2)[0]) < 1e-12
    x = rng.standard_normal(50)
    assert abs(O.rank_correlation(x, x)[1] - 1.0) < 1e-12
    assert abs(O.rank_correlation(x, -x)[1] + 1.0) < 1e-12
    assert abs(O.rank_correlation(x, np.exp(x))[1] - 1.0) < 1e-12   # monotone map keeps ranks


# ----------------------------------------------------------------------------
# low-bit middle streams

def pin_quant_closed_forms(O):
    # a constant group has nothing to resolve: code 0, scale 0, exact
    codes, scale, lo = O.quantize_asym(np.full((64, 5), 1.5, dtype=np.float32), 4, axis=0)
    assert np.all(codes == 0) and np.all(scale == 0) and np.all(lo == np.float32(1.5))
    assert np.all(O.dequantize(codes, scale, lo) == 1.5)
    rng = np.random.default_rng(40)
    for bits in (2, 4, 8):
        top = 2 ** bits - 1
        # values on the grid lo + k * step (exact in float32), both ends present
        k = rng.integers(0, top + 1, size=(64, 7))
        k[3], k[11] = 0, top
        x = (-1.0 + k * 0.125).astype(np.float32)
        codes, scale, lo = O.quantize_asym(x, bits, axis=0)
        assert np.array_equal(codes.astype(np.int64), k), bits
        assert np.all(scale == np.float32(0.125)) and np.all(lo == np.float32(-1.0))
        assert np.array_equal(O.dequantize(codes, scale, lo), x.astype(np.float64))


def pin_quant_nearest_level(O):
    rng = np.random.default_rng(41)
    for bits in (2, 4, 8):
        top = 2 ** bits - 1
        x = _bits_to_f64(_f32_to_bf16_bits(rng.standard_normal((64, 9)) * 3.0)).numpy().astype(np.float32)
        codes, scale, lo = O.quantize_asym(x, bits, axis=0)
        sc = scale.astype(np.float64)[0]
        lo64 = lo.astype(np.float64)[0]
        assert np.all(codes <= top)
        for col in range(x.shape[1]):
            levels = lo64[col] + np.arange(top + 1) * sc[col]
            dist = np.abs(x[:, col, None].astype(np.float64) - levels[None, :])
            chosen = dist[np.arange(64), codes[:, col].astype(np.int64)]
            assert np.all(chosen <= dist.min(axis=1) + 1e-6 * sc[col]), (bits, col)
            assert np.all(chosen <= 0.5 * sc[col] * (1 + 1e-5)), (bits, col)
            # the group's extremes land on the end levels
            assert codes[np.argmin(x[:, col]), col] == 0
            assert codes[np.argmax(x[:, col]), col] == top


def pin_quant_middle_groups(O):
    rng = np.random.default_rng(42)
    c, t_mid, group = 16, 3 * 64 + 21, 64
    k_bits = _f32_to_bf16_bits(rng.standard_normal((t_mid, c)))
    v_bits = _f32_to_bf16_bits(rng.standard_normal((t_mid, 128)))
    for bits in (4, 8):
        top = 2 ** bits - 1
        qm = O.quantize_middle(k_bits, v_bits, bits, group)
        assert qm["k_codes"].shape == (3 * group, c)
        assert np.array_equal(qm["k_stage"], k_bits[3 * group:])   # incomplete group exact
        kx = _bits_to_f64(k_bits).numpy()
        for g in range(3):
            rows = kx[g * group:(g + 1) * group]
            codes = qm["k_codes"][g * group:(g + 1) * group]
            for ch in range(c):    # per channel over the group's rows
                assert codes[np.argmin(rows[:, ch]), ch] == 0
                assert codes[np.argmax(rows[:, ch]), ch] == top
        vx = _bits_to_f64(v_bits).numpy()
        for r in range(t_mid):     # per token over its channels
            assert qm["v_codes"][r, np.argmin(vx[r])] == 0
            assert qm["v_codes"][r, np.argmax(vx[r])] == top


def pin_quant_ties_to_even(O):
    # values exactly half-way between two levels (float32-exact: the quotient
    # (x - lo) / scale is k + 1/2 with no rounding) take the even code, the
    # IEEE default rounding of the reading the low-bit streams follow
    for bits in (2, 4, 8):
        top = 2 ** bits - 1
        k = np.arange(top)
        for lo, step in ((0.0, 1.0), (-3.0, 0.25)):
            x = lo + np.concatenate([[0.0, float(top)], k + 0.5]) * step
            want = np.concatenate([[0, top], k + (k & 1)])
            for axis, arr in ((0, x[:, None]), (1, x[None, :])):
                codes, scale, lo_q = O.quantize_asym(arr.astype(np.float32), bits, axis=axis)
                assert np.all(scale == np.float32(step)) and np.all(lo_q == np.float32(lo))
                assert np.array_equal(codes.reshape(-1).astype(np.int64), want), (bits, lo, axis)


def pin_pack_q_contents(O):
    # grid-exact K/V (both ends of every grid present), coded by position,
    # channel, batch row and head: every (b, live h) of the low-bit pack must
    # give back exactly that pair's own middle -- its kept K channels of the
    # complete groups from the codes, the open group's K rows as bf16, and
    # its V rows from the codes -- and a dead head holds nothing
    n_sink, window, d, group = 3, 5, 128, 64
    batch, n_kv, kept = 2, 3, [32, 0, 64]
    rng = np.random.default_rng(46)
    kept_idx = np.full((n_kv, d), -1, dtype=np.int64)
    for h, c in enumerate(kept):
        kept_idx[h, :c] = np.sort(rng.choice(d, size=c, replace=False))
    t_mid = 2 * group + 19
    ctx_len = n_sink + t_mid + window
    t = np.arange(ctx_len)[None, None, :, None]
    ch = np.arange(d)[None, None, None, :]
    bb = np.arange(batch)[:, None, None, None]
    hh = np.arange(n_kv)[None, :, None, None]
    for bits in (4, 8):
        top = 2 ** bits - 1
        lvl_k = np.broadcast_to((3 * t + 5 * ch + 7 * bb + 11 * hh) % (top + 1),
                                (batch, n_kv, ctx_len, d)).copy()
        lvl_v = np.broadcast_to((5 * t + 3 * ch + 11 * bb + 7 * hh) % (top + 1),
                                (batch, n_kv, ctx_len, d)).copy()
        for b in range(batch):
            for h in range(n_kv):
                for g in range(t_mid // group):       # K: each channel spans its group's grid
                    r0 = n_sink + g * group
                    lvl_k[b, h, r0 + (b + h) % 32, :] = 0
                    lvl_k[b, h, r0 + 32 + (b + 2 * h) % 32, :] = top
                for r in range(ctx_len):              # V: each row spans its grid
                    lvl_v[b, h, r, (r + b) % 64] = 0
                    lvl_v[b, h, r, 64 + (r + h) % 64] = top
        lo_k = -2.0 + 0.25 * bb + 0.5 * hh
        lo_v = -1.5 + 0.5 * bb + 0.25 * hh
        k = _f32_to_bf16_bits(lo_k + lvl_k * 0.125)       # multiples of 1/8 below 32: exact
        v = _f32_to_bf16_bits(lo_v + lvl_v * 0.125)
        ref = O.pack_reference_q(k, v, kept, kept_idx, n_sink, window, bits, group)
        assert ref["mid_q"][1] is None, bits
        mids = np.arange(n_sink, n_sink + t_mid)
        n_full = (t_mid // group) * group
        for h in (0, 2):
            idx = kept_idx[h, :kept[h]]
            assert len(ref["mid_q"][h]) == batch
            for b in range(batch):
                m = ref["mid_q"][h][b]
                want_k = _bits_to_f64(k[b, h][mids][:, idx]).numpy()
                want_v = _bits_to_f64(v[b, h][mids]).numpy()
                kc = m["k_codes"].astype(np.float64).reshape(-1, group, kept[h])
                got_k = (kc * m["k_scale"].astype(np.float64)[:, None, :]
                         + m["k_lo"].astype(np.float64)[:, None, :]).reshape(n_full, kept[h])
                assert np.array_equal(got_k, want_k[:n_full]), (bits, h, b)
                assert np.array_equal(m["k_stage"], k[b, h][mids][n_full:][:, idx]), (bits, h, b)
                got_v = (m["v_codes"].astype(np.float64) * m["v_scale"].astype(np.float64)[:, None]
                         + m["v_lo"].astype(np.float64)[:, None])
                assert np.array_equal(got_v, want_v), (bits, h, b)


def _grid_context(rng, batch, n_kv, ctx_len, d, bits, mid_lo, mid_hi, group):
    """K, V bits whose middle rows [mid_lo, mid_hi) lie on per-group
    (K, per channel) and per-row (V) grids with both ends present, so that
    quantization is lossless; other rows are generic."""
    top = 2 ** bits - 1
    k = rng.standard_normal((batch, n_kv, ctx_len, d))
    v = rng.standard_normal((batch, n_kv, ctx_len, d))
    n_groups = (mid_hi - mid_lo) // group
    for g in range(n_groups):
        r0 = mid_lo + g * group
        lvl = rng.integers(0, top + 1, size=(batch, n_kv, group, d))
        lvl[:, :, 0], lvl[:, :, 1] = 0, top
        k[:, :, r0:r0 + group] = -2.0 + lvl * 0.25
    lvl = rng.integers(0, top + 1, size=(batch, n_kv, mid_hi - mid_lo, d))
    lvl[..., 0], lvl[..., 1] = 0, top
    v[:, :, mid_lo:mid_hi] = -1.0 + lvl * 0.125
    return _f32_to_bf16_bits(k), _f32_to_bf16_bits(v)


def pin_decode_q_grid_exact(O):
    rng = np.random.default_rng(43)
    n_sink, window, group, d = 4, 8, 64, 128
    for bits in (4, 8):
        ctx_len = n_sink + 2 * group + 37 + window     # two full groups + an open one
        k, v = _grid_context(rng, 2, 2, ctx_len, d, bits, n_sink, n_sink + 2 * group + 37, group)
        q = _f32_to_bf16_bits(rng.standard_normal((2, 4, d)))
        mask = _random_mask(rng, 2, d, 32)
        mask[1] = 0                                     # one dead head
        mask[0, :] = 1                                  # one head keeps every channel
        ref = O.decode(q, k, v, mask, n_sink, window)
        got = O.decode_q(q, k, v, mask, n_sink, window, bits, group)
        assert np.max(np.abs(got - ref)) < 1e-12, bits
    # each stream on its own: with the other one grid-exact, quantizing
    # generic values changes the result
    ctx_len = n_sink + 2 * group + window
    k2, v2 = _grid_context(rng, 2, 2, ctx_len, d, 2, n_sink, n_sink + 2 * group, group)
    kg = _f32_to_bf16_bits(rng.standard_normal((2, 2, ctx_len, d)))
    vg = _f32_to_bf16_bits(rng.standard_normal((2, 2, ctx_len, d)))
    q = _f32_to_bf16_bits(rng.standard_normal((2, 4, d)) * 2.0)
    mask = np.ones((2, d), dtype=np.uint8)
    assert np.max(np.abs(O.decode_q(q, k2, v2, mask, n_sink, window, 2, group)
                         - O.decode(q, k2, v2, mask, n_sink, window))) < 1e-12
    for k, v, what in ((kg, v2, "K"), (k2, vg, "V")):
        diff = np.max(np.abs(O.decode_q(q, k, v, mask, n_sink, window, 2, group)
                             - O.decode(q, k, v, mask, n_sink, window)))
        assert diff > 1e-3, what


def pin_traffic_bytes_q(O):
    rng = np.random.default_rng(44)
    n_sink, window, d, group = 4, 8, 128, 64
    for bits in (4, 8):
        for ctx_len in (5, n_sink + window, n_sink + window + 63, n_sink + window + 64 + 29):
            kept = [32, 0, 64]
            mask = np.zeros((3, d), dtype=np.uint8)
            for h, c in enumerate(kept):
                mask[h, np.sort(rng.choice(d, size=c, replace=False))] = 1
            kept_idx = np.full((3, d), -1, dtype=np.int64)
            for h in range(3):
                kept_idx[h, :kept[h]] = np.flatnonzero(mask[h])
            k = _f32_to_bf16_bits(rng.standard_normal((2, 3, ctx_len, d)))
            ref = O.pack_reference_q(k, k, kept, kept_idx, n_sink, window, bits, group)
            n_full = min(ctx_len, n_sink) + max(0, min(window, ctx_len - n_sink))
            total = 2 * 6 * d * 2 + 2 * 6 * d * 4 + 2 * 2 * 3 * n_full * d * 2
            for per_b in ref["mid_q"]:
                for m in per_b or []:
                    total += (m["k_codes"].size + m["v_codes"].size) * bits // 8
                    total += (m["k_scale"].nbytes + m["k_lo"].nbytes + m["k_stage"].nbytes
                              + m["v_scale"].nbytes + m["v_lo"].nbytes)
            assert O.decode_traffic_bytes_q(2, 6, 3, d, ctx_len, n_sink, window, kept, bits,
                                            group) == total, (bits, ctx_len)


ALL_PINS = [
    pin_mask_page_procedure,
    pin_mask_closed_forms,
    pin_mask_invariants,
    pin_mask_bruteforce,
    pin_pack_layout,
    pin_pack_round_trip,
    pin_decode_dense_matches_sdpa,
    pin_decode_masked_matches_sdpa,
    pin_decode_closed_forms,
    pin_decode_bruteforce,
    pin_cache_bytes,
    pin_traffic_bytes,
    pin_analysis,
    pin_quant_closed_forms,
    pin_quant_nearest_level,
    pin_quant_middle_groups,
    pin_quant_ties_to_even,
    pin_pack_q_contents,
    pin_decode_q_grid_exact,
    pin_traffic_bytes_q,
]
