"""Ragged batches: per-row context lengths and per-row appends, against the
CPU oracle applied to each row's own tokens (bit-exact cache rows,
attention within 2e-3 + 1e-2 |oracle|)."""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import (assert_cache_matches, assert_close, make_cache, mask_with_counts,
                             random_bf16)

pytestmark = pytest.mark.gpu
DEV = "cuda"
COUNTS = [32, 0, 64, 128, 8]


def case(*args):
    print("CASE", *args, flush=True)


def _check_rows(cache, k, v, q, mask, lengths, out, n_sink, window):
    kh, vh, qh = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    for b, length in enumerate(lengths):
        if length == 0:
            assert np.all(out[b] == 0.0)
            continue
        pairs = [(b, h) for h in range(mask.shape[0])]
        sel_k = np.stack([kh[b, h, :length] for h in range(mask.shape[0])])[:, None]
        sel_v = np.stack([vh[b, h, :length] for h in range(mask.shape[0])])[:, None]
        assert_cache_matches(cache, sel_k, sel_v, mask, pairs=pairs)
        ref = oracle.decode(qh[b:b + 1], kh[b:b + 1, :, :length], vh[b:b + 1, :, :length], mask,
                            n_sink, window)
        assert_close(out[b:b + 1], ref, f"row {b} length {length}")


@pytest.mark.parametrize("window", [16, 64])
def test_ragged_prefill_then_steps(window):
    n_sink, group, max_ctx = 4, 4, 1200
    lengths = [1, 3, 4, 19, 20, 21, 300, 1000]
    batch = len(lengths)
    mask = mask_with_counts(np.random.default_rng(window), COUNTS)
    n_kv = mask.shape[0]
    cache = make_cache(mask, batch, n_kv * group, n_sink, window, max_ctx)
    gen = torch.Generator(device=DEV).manual_seed(window)
    full = max_ctx
    k = random_bf16((batch, n_kv, full, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, full, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    n_pre = max(lengths)
    case("ragged prefill", window)
    row_pos = torch.zeros(batch, dtype=torch.int64, device=DEV)
    row_cnt = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    dac.leank_pack_k_rows(cache, k[:, :, :n_pre].contiguous(), v[:, :, :n_pre].contiguous(),
                          row_pos, row_cnt)
    ctx = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    out = dac.leank_decode_attn_rows(cache, q, ctx, max_ctx_len=max(lengths))
    torch.cuda.synchronize()
    _check_rows(cache, k, v, q, mask, lengths, out.cpu().numpy(), n_sink, window)

    # decode steps: most rows append one token per step, some skip steps
    lens = list(lengths)
    rng = np.random.default_rng(5)
    for step in range(40):
        counts = [int(rng.random() < 0.8) for _ in range(batch)]
        chunk = torch.stack([k[b, :, lens[b]:lens[b] + 1] for b in range(batch)])
        vchunk = torch.stack([v[b, :, lens[b]:lens[b] + 1] for b in range(batch)])
        pos = torch.tensor(lens, dtype=torch.int64, device=DEV)
        cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
        dac.leank_pack_k_rows(cache, chunk.contiguous(), vchunk.contiguous(), pos, cnt)
        lens = [lens[b] + counts[b] for b in range(batch)]
        if step % 13 == 12 or step == 39:
            case("ragged step", window, step)
            ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
            out = dac.leank_decode_attn_rows(cache, q, ctx, max_ctx_len=max(lens))
            torch.cuda.synchronize()
            _check_rows(cache, k, v, q, mask, lens, out.cpu().numpy(), n_sink, window)


def test_ragged_bulk_appends_in_chunks():
    # rows at different lengths append different chunk sizes, some larger than the window
    n_sink, window, group, max_ctx = 3, 16, 2, 400
    mask = mask_with_counts(np.random.default_rng(9), COUNTS)
    n_kv = mask.shape[0]
    batch = 4
    cache = make_cache(mask, batch, n_kv * group, n_sink, window, max_ctx)
    gen = torch.Generator(device=DEV).manual_seed(9)
    k = random_bf16((batch, n_kv, max_ctx, 128), gen)
    v = random_bf16((batch, n_kv, max_ctx, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    lens = [0, 0, 0, 0]
    rng = np.random.default_rng(1)
    for rnd in range(6):
        n_new = int(rng.choice([5, 16, 17, 40]))
        counts = [int(rng.integers(0, n_new + 1)) for _ in range(batch)]
        counts = [min(c, max_ctx - lens[b]) for b, c in enumerate(counts)]
        case("ragged chunks", rnd, n_new, counts)
        kc = torch.zeros((batch, n_kv, n_new, 128), dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        for b in range(batch):
            kc[b, :, :counts[b]] = k[b, :, lens[b]:lens[b] + counts[b]]
            vc[b, :, :counts[b]] = v[b, :, lens[b]:lens[b] + counts[b]]
        dac.leank_pack_k_rows(cache, kc, vc, torch.tensor(lens, dtype=torch.int64, device=DEV),
                              torch.tensor(counts, dtype=torch.int32, device=DEV))
        lens = [lens[b] + counts[b] for b in range(batch)]
        ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
        out = dac.leank_decode_attn_rows(cache, q, ctx, max_ctx_len=max(max(lens), 1))
        torch.cuda.synchronize()
        _check_rows(cache, k, v, q, mask, lens, out.cpu().numpy(), n_sink, window)


def test_rows_outside_the_cache_are_left_unchanged():
    n_sink, window, max_ctx = 2, 8, 50
    mask = mask_with_counts(np.random.default_rng(2), [32, 0])
    cache = make_cache(mask, 2, 2, n_sink, window, max_ctx)
    gen = torch.Generator(device=DEV).manual_seed(2)
    k = random_bf16((2, 2, 30, 128), gen)
    v = random_bf16((2, 2, 30, 128), gen)
    case("ragged out of range")
    dac.leank_pack_k(cache, k, v)
    torch.cuda.synchronize()
    before = [t.clone() for t in (cache.k_sl, cache.v_sl, cache.k_prun, cache.v_mid)]
    kn = random_bf16((2, 2, 5, 128), gen)
    bad_pos = torch.tensor([48, -3], dtype=torch.int64, device=DEV)   # 48 + 5 > 50; negative
    dac.leank_pack_k_rows(cache, kn, kn, bad_pos)
    torch.cuda.synchronize()
    for a, b in zip(before, (cache.k_sl, cache.v_sl, cache.k_prun, cache.v_mid)):
        assert torch.equal(a, b)
