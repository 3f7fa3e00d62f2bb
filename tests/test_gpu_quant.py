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


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n_sink,window", [(4, 16), (6, 0)])
def test_chunked_appends_match_bulk(bits, n_sink, window):
    """Appends of several tokens into a non-empty cache (token by token in
    one kernel, across group completions) leave the cache the bulk packing
    of the same tokens would."""
    batch, t0 = 2, n_sink + window + 30
    chunks = [5, 64, 1, 130, 17]
    total = t0 + sum(chunks)
    mask = mask_with_counts(np.random.default_rng(31 + bits), COUNTS)
    n_kv = mask.shape[0]
    cache = make_qcache(mask, batch, n_kv * 2, n_sink, window, total, bits)
    gen = torch.Generator(device=DEV).manual_seed(41 + bits + window)
    k = random_bf16((batch, n_kv, total, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, total, 128), gen)
    case("quant chunked appends", bits, n_sink, window)
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    kh, vh = bf16_bits(k), bf16_bits(v)
    pos = t0
    for n in chunks:
        dac.leank_pack_k(cache, k[:, :, pos:pos + n].contiguous(), v[:, :, pos:pos + n].contiguous(),
                         pos0=pos)
        pos += n
        torch.cuda.synchronize()
        assert_quant_cache_matches(cache, kh[:, :, :pos], vh[:, :, :pos], mask)


def _ragged_qcache(bits, lens, n_sink, window, max_ctx, seed, counts=(32, 0, 64, 8), group=2):
    """A low-bit cache whose rows hold lens[b] tokens, built with ragged
    appends from empty in two rounds; returns the cache, the mask and the
    full per-row token streams."""
    batch = len(lens)
    mask = mask_with_counts(np.random.default_rng(seed), list(counts))
    n_kv = mask.shape[0]
    cache = make_qcache(mask, batch, n_kv * group, n_sink, window, max_ctx, bits)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    width = max(lens) + 2
    k = random_bf16((batch, n_kv, width, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, width, 128), gen)
    first = [min(n, 70 + 13 * b) for b, n in enumerate(lens)]
    for start, cnt in ((np.zeros(batch, np.int64), first),
                       (np.array(first, np.int64), [n - f for n, f in zip(lens, first)])):
        n_new = max(max(cnt), 1)
        kk = torch.zeros((batch, n_kv, n_new, 128), dtype=torch.bfloat16, device=DEV)
        vv = torch.zeros_like(kk)
        for b in range(batch):
            kk[b, :, :cnt[b]] = k[b, :, start[b]:start[b] + cnt[b]]
            vv[b, :, :cnt[b]] = v[b, :, start[b]:start[b] + cnt[b]]
        dac.leank_pack_k_rows(cache, kk, vv, torch.from_numpy(start).to(DEV),
                              torch.tensor(cnt, dtype=torch.int32, device=DEV))
    return cache, mask, k, v


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n_sink,window", [(4, 16), (0, 8), (5, 0)])
def test_ragged_appends_match_bulk(bits, n_sink, window):
    """leank_pack_k_rows on a low-bit cache: each row holds what the bulk
    packing of its own tokens gives."""
    lens = [0, 1, n_sink + window + 63, n_sink + window + 64, 300]
    case("quant ragged appends", bits, n_sink, window)
    cache, mask, k, v = _ragged_qcache(bits, lens, n_sink, window, 320, 53 + bits + window)
    torch.cuda.synchronize()
    kh, vh = bf16_bits(k), bf16_bits(v)
    for b, n in enumerate(lens):
        if n:
            assert_quant_cache_matches(cache, kh[b:b + 1, :, :n], vh[b:b + 1, :, :n], mask, rows=[b])


# ---------------------------------------------------------------- attention over low-bit streams

def _oracle_q(q, k, v, mask, n_sink, window, bits, pairs=None):
    return oracle.decode_q(bf16_bits(q), bf16_bits(k), bf16_bits(v), mask, n_sink, window, bits,
                           pairs=pairs)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("ctx", [3, 20, 20 + 64, 20 + 64 + 37, 20 + 5 * 64 + 1, 1000])
def test_decode_matches_oracle(bits, group, ctx):
    n_sink, window, batch = 4, 16, 2
    mask = mask_with_counts(np.random.default_rng(ctx + group), [32, 0, 64, 128, 8, 40])
    n_kv = mask.shape[0]
    cache = make_qcache(mask, batch, n_kv * group, n_sink, window, 1024, bits)
    gen = torch.Generator(device=DEV).manual_seed(ctx * 3 + bits)
    k = random_bf16((batch, n_kv, ctx, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, ctx, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    case("quant decode", bits, group, ctx)
    dac.leank_pack_k(cache, k, v)
    out = dac.leank_decode_attn(cache, q)
    again = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    assert_close(out.cpu().numpy(), _oracle_q(q, k, v, mask, n_sink, window, bits),
                 f"bits {bits} G {group} ctx {ctx}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [4, 7])
def test_decode_channel_scales(bits, group):
    """K channels whose magnitudes differ by orders of magnitude (log-normal
    scales): the per-channel group scales folded into the query span as
    wide a range."""
    n_sink, window, batch, ctx = 4, 16, 2, 20 + 7 * 64 + 9
    mask = mask_with_counts(np.random.default_rng(5), [32, 64, 128])
    cache = make_qcache(mask, batch, 3 * group, n_sink, window, ctx, bits)
    gen = torch.Generator(device=DEV).manual_seed(17 + bits)
    rng = np.random.default_rng(23)
    ch_scale = torch.from_numpy(np.exp(rng.normal(0.0, 1.5, size=128)).astype(np.float32)).to(DEV)
    k = (random_bf16((batch, 3, ctx, 128), gen).float() * ch_scale).to(torch.bfloat16)
    v = random_bf16((batch, 3, ctx, 128), gen)
    q = random_bf16((batch, 3 * group, 128), gen, scale=0.3)
    case("quant decode channel scales", bits, group)
    dac.leank_pack_k(cache, k, v)
    out = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), _oracle_q(q, k, v, mask, n_sink, window, bits),
                 f"channel scales bits {bits} G {group}")


@pytest.mark.parametrize("bits", [4, 8])
def test_decode_large_values(bits):
    """Wide value ranges: codes and the folded minimum over large magnitudes."""
    n_sink, window, batch, ctx = 4, 16, 1, 400
    mask = mask_with_counts(np.random.default_rng(3), [32, 64])
    cache = make_qcache(mask, batch, 8, n_sink, window, ctx, bits)
    gen = torch.Generator(device=DEV).manual_seed(11)
    k = random_bf16((batch, 2, ctx, 128), gen, scale=6.0)
    v = (random_bf16((batch, 2, ctx, 128), gen, scale=30.0).float() + 100.0).to(torch.bfloat16)
    q = random_bf16((batch, 8, 128), gen, scale=0.5)
    case("quant decode large", bits)
    dac.leank_pack_k(cache, k, v)
    out = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), _oracle_q(q, k, v, mask, n_sink, window, bits), "large")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n_sink,window", [(4, 16), (6, 0)])
def test_step_on_quant_cache(bits, n_sink, window):
    """leank_decode_step on a low-bit cache across group completions."""
    batch, group, t0, steps = 2, 4, n_sink + window + 60, 70
    mask = mask_with_counts(np.random.default_rng(window + bits), COUNTS)
    n_kv = mask.shape[0]
    cache = make_qcache(mask, batch, n_kv * group, n_sink, window, t0 + steps, bits)
    gen = torch.Generator(device=DEV).manual_seed(window * 5 + bits)
    k = random_bf16((batch, n_kv, t0 + steps, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, t0 + steps, 128), gen)
    q = random_bf16((steps, batch, n_kv * group, 128), gen)
    case("quant step", bits, n_sink, window)
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    outs = []
    for s in range(steps):
        outs.append(dac.leank_decode_step(cache, q[s], k[:, :, t0 + s].contiguous(),
                                          v[:, :, t0 + s].contiguous()))
    torch.cuda.synchronize()
    kh, vh = bf16_bits(k), bf16_bits(v)
    assert_quant_cache_matches(cache, kh, vh, mask)
    for s in (0, 3, 4, 5, steps - 1):
        ref = oracle.decode_q(bf16_bits(q[s]), kh[:, :, :t0 + s + 1], vh[:, :, :t0 + s + 1], mask,
                              n_sink, window, bits)
        assert_close(outs[s].cpu().numpy(), ref, f"step {s}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [1, 4])
def test_ragged_decode_on_quant_cache(bits, group):
    """leank_decode_attn_rows: each row attends over its own length."""
    n_sink, window = 4, 16
    lens = [1, 20, 20 + 64, 20 + 64 + 37, 20 + 5 * 64 + 1]
    case("quant ragged decode", bits, group)
    cache, mask, k, v = _ragged_qcache(bits, lens, n_sink, window, 420, 61 + bits, group=group)
    n_kv = mask.shape[0]
    gen = torch.Generator(device=DEV).manual_seed(67 + bits)
    q = random_bf16((len(lens), n_kv * group, 128), gen)
    out = dac.leank_decode_attn_rows(cache, q, torch.tensor(lens, dtype=torch.int32, device=DEV),
                                     max_ctx_len=max(lens))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, n in enumerate(lens):
        ref = _oracle_q(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], mask, n_sink, window, bits)
        assert_close(got[b:b + 1], ref, f"ragged decode bits {bits} G {group} row {b}")


@pytest.mark.parametrize("bits", [4, 8])
def test_ragged_step_on_quant_cache(bits):
    """leank_decode_step_rows: row b appends at row_pos[b] and attends over
    row_pos[b] + 1 tokens; rows whose position is out of range are left as
    they were and get zeros.  Rows cross group completions at different
    steps."""
    n_sink, window, group = 4, 16, 2
    lens = [1, 40, 83, 84, 150, 7]
    max_ctx_len = 160
    case("quant ragged step", bits)
    cache, mask, k, v = _ragged_qcache(bits, lens, n_sink, window, 200, 71 + bits, group=group)
    n_kv = mask.shape[0]
    kh, vh = bf16_bits(k), bf16_bits(v)
    gen = torch.Generator(device=DEV).manual_seed(73 + bits)
    steps = 70
    extra_k = random_bf16((steps, len(lens), n_kv, 128), gen, scale=2.0)
    extra_v = random_bf16((steps, len(lens), n_kv, 128), gen)
    pos = list(lens)
    pos[5] = -1  # a row that takes no part
    hist_k = [kh[b, :, :n] for b, n in enumerate(lens)]
    hist_v = [vh[b, :, :n] for b, n in enumerate(lens)]
    for s in range(steps):
        q = random_bf16((len(lens), n_kv * group, 128), gen)
        out = dac.leank_decode_step_rows(cache, q, extra_k[s], extra_v[s],
                                         torch.tensor(pos, dtype=torch.int64, device=DEV),
                                         max_ctx_len=max_ctx_len)
        for b in range(len(lens)):
            if 0 <= pos[b] < max_ctx_len:
                hist_k[b] = np.concatenate([hist_k[b], bf16_bits(extra_k[s][b])[:, None]], axis=1)
                hist_v[b] = np.concatenate([hist_v[b], bf16_bits(extra_v[s][b])[:, None]], axis=1)
        if s in (0, 1, 43, 44, steps - 1):
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for b in range(len(lens)):
                if not 0 <= pos[b] < max_ctx_len:
                    assert not got[b].any(), (s, b)
                    assert_quant_cache_matches(cache, hist_k[b][None], hist_v[b][None], mask, rows=[b])
                    continue
                ref = oracle.decode_q(bf16_bits(q[b:b + 1]), hist_k[b][None], hist_v[b][None], mask,
                                      n_sink, window, bits)
                assert_close(got[b:b + 1], ref, f"ragged step bits {bits} step {s} row {b}")
                assert_quant_cache_matches(cache, hist_k[b][None], hist_v[b][None], mask, rows=[b])
        for b in range(len(lens)):
            if 0 <= pos[b] < max_ctx_len:
                pos[b] += 1


@pytest.mark.parametrize("bits", [4, 8])
def test_full_workload_quant_sampled(bits):
    from synthetic import alpha_for, get_config, make_kv, make_q

    cfg = get_config("llama_b64_4k")
    om, okc, oki = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
    case("quant full workload", bits)
    cache = dac.LayerCache(okc[0].tolist(), torch.from_numpy(oki[0]).to(DEV), cfg.batch,
                           cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, cfg.ctx,
                           quant_bits=bits)
    k, v = make_kv(cfg, 0, device=DEV)
    t0 = cfg.ctx - 2
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    rng = np.random.default_rng(bits)
    pairs = sorted({(int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_q_heads)))
                    for _ in range(16)} | {(0, 0), (cfg.batch - 1, cfg.n_q_heads - 1)})
    kh, vh = bf16_bits(k), bf16_bits(v)
    for s in range(2):
        q = make_q(cfg, 0, step=s + 1, device=DEV)
        out = dac.leank_decode_step(cache, q, k[:, :, t0 + s].contiguous(),
                                    v[:, :, t0 + s].contiguous())
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = oracle.decode_q(bf16_bits(q), kh[:, :, :t0 + s + 1], vh[:, :, :t0 + s + 1], om[0],
                              cfg.n_sink, cfg.window, bits, pairs=pairs)
        assert_close(np.stack([got[b, j] for b, j in pairs]), ref, f"bits {bits} step {s}")
