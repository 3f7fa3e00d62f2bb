"""Low-bit middle streams (K per channel over 64-row groups, V per token,
4 and 8 bits) against the CPU oracle: every code, scale, minimum and staged
row bit for bit, and attention over the dequantized middle within
2e-3 + 1e-2 |oracle|."""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import (assert_close, assert_quant_cache_matches, kept_from_mask,
                             mask_with_counts, random_bf16)

pytestmark = pytest.mark.gpu
DEV = "cuda"
COUNTS = [32, 0, 64, 128, 8]


def case(*args):
    print("CASE", *args, flush=True)


def make_qcache(mask, batch, n_q, n_sink, window, max_ctx, bits):
    kept_count, kept_idx = kept_from_mask(mask)
    return dac.LayerCache(kept_count.tolist(), torch.from_numpy(kept_idx).to(DEV), batch, n_q,
                          mask.shape[0], n_sink, window, max_ctx, device=DEV, quant_bits=bits)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n_sink,window,t0", [(4, 16, 300), (4, 16, 4 + 16 + 128),
                                              (0, 32, 250), (5, 0, 200), (4, 64, 40)])
def test_bulk_prefill_matches_oracle(bits, n_sink, window, t0):
    batch = 2
    mask = mask_with_counts(np.random.default_rng(t0 + bits), COUNTS)
    n_kv = mask.shape[0]
    cache = make_qcache(mask, batch, n_kv * 2, n_sink, window, t0 + 8, bits)
    gen = torch.Generator(device=DEV).manual_seed(t0 + window)
    k = random_bf16((batch, n_kv, t0, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, t0, 128), gen)
    case("quant bulk", bits, n_sink, window, t0)
    dac.leank_pack_k(cache, k, v)
    torch.cuda.synchronize()
    assert_quant_cache_matches(cache, bf16_bits(k), bf16_bits(v), mask)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n_sink,window", [(4, 16), (6, 0), (0, 8)])
def test_single_token_appends_match_bulk(bits, n_sink, window):
    """Prefill, then one token per call across several group completions."""
    batch, t0, steps = 2, n_sink + window + 50, 150
    mask = mask_with_counts(np.random.default_rng(bits + window), COUNTS)
    n_kv = mask.shape[0]
    cache = make_qcache(mask, batch, n_kv * 2, n_sink, window, t0 + steps, bits)
    gen = torch.Generator(device=DEV).manual_seed(bits * 7 + window)
    k = random_bf16((batch, n_kv, t0 + steps, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, t0 + steps, 128), gen)
    case("quant appends", bits, n_sink, window)
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    kh, vh = bf16_bits(k), bf16_bits(v)
    for s in range(steps):
        pos = t0 + s
        dac.leank_pack_k(cache, k[:, :, pos:pos + 1].contiguous(), v[:, :, pos:pos + 1].contiguous())
        if s in (13, 14, 77, steps - 1):
            torch.cuda.synchronize()
            assert_quant_cache_matches(cache, kh[:, :, :pos + 1], vh[:, :, :pos + 1], mask)


@pytest.mark.parametrize("bits", [4, 8])
def test_appends_from_empty(bits):
    n_sink, window, batch, steps = 3, 5, 1, 140
    mask = mask_with_counts(np.random.default_rng(9), [64, 0, 8])
    cache = make_qcache(mask, batch, 6, n_sink, window, steps, bits)
    gen = torch.Generator(device=DEV).manual_seed(bits)
    k = random_bf16((batch, 3, steps, 128), gen)
    v = random_bf16((batch, 3, steps, 128), gen)
    case("quant appends from empty", bits)
    for pos in range(steps):
        dac.leank_pack_k(cache, k[:, :, pos:pos + 1].contiguous(), v[:, :, pos:pos + 1].contiguous())
    torch.cuda.synchronize()
    assert_quant_cache_matches(cache, bf16_bits(k), bf16_bits(v), mask)


def test_quant_pack_rejections():
    mask = mask_with_counts(np.random.default_rng(2), [32, 0])
    cache = make_qcache(mask, 1, 2, 4, 8, 100, 4)
    gen = torch.Generator(device=DEV).manual_seed(2)
    k = random_bf16((1, 2, 20, 128), gen)
    case("quant rejections")
    dac.leank_pack_k(cache, k, k)
    with pytest.raises(dac.LeankError) as err:   # chunked append into a non-empty cache
        dac.leank_pack_k(cache, k[:, :, :2].contiguous(), k[:, :, :2].contiguous())
    assert err.value.status == dac._lib.EUNSUPPORTED
    with pytest.raises(dac.LeankError) as err:
        dac.leank_pack_k_rows(cache, k[:, :, :1].contiguous(), k[:, :, :1].contiguous(),
                              torch.zeros(1, dtype=torch.int64, device=DEV))
    assert err.value.status == dac._lib.EUNSUPPORTED
