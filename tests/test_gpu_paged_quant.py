"""Paged low-bit middle (one 64-row K group per page, from a pool through a
block table) against the CPU oracle: every code, scale, minimum and staged
row read back through the table bit for bit, attention within 2e-3 +
1e-2 |oracle|, pages outside the table untouched."""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import (assert_close, assert_quant_cache_matches, kept_from_mask,
                             mask_with_counts, random_bf16, shuffled_block_table)

pytestmark = pytest.mark.gpu
DEV = "cuda"
COUNTS = [32, 0, 64, 128, 8]
SENTINEL = 0xA5


def case(*args):
    print("CASE", *args, flush=True)


def make_paged_q(mask, batch, n_q, n_sink, window, max_ctx, bits, seed, spare=5):
    kept_count, kept_idx = kept_from_mask(mask)
    mid_cap = max(0, max_ctx - n_sink - window)
    ppr = -(-mid_cap // 64)
    n_pages = batch * ppr + spare
    table = shuffled_block_table(np.random.default_rng(seed), batch, ppr, n_pages)
    cache = dac.LayerCache(kept_count.tolist(), torch.from_numpy(kept_idx).to(DEV), batch, n_q,
                           mask.shape[0], n_sink, window, max_ctx, device=DEV, n_pages=n_pages,
                           block_table=table, quant_bits=bits)
    cache.pool.view(torch.uint8).fill_(SENTINEL)
    return cache


def unused_pages_untouched(cache):
    used = set(cache.block_table.cpu().numpy().ravel().tolist())
    pb = cache.desc.page_bytes
    pool = cache.pool.view(torch.uint8).cpu().numpy()
    for page in range(cache.desc.n_pages):
        if page not in used:
            assert np.all(pool[page * pb:(page + 1) * pb] == SENTINEL), page


def _oracle_q(q, k, v, mask, n_sink, window, bits):
    return oracle.decode_q(bf16_bits(q), bf16_bits(k), bf16_bits(v), mask, n_sink, window, bits)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [1, 4, 7])
@pytest.mark.parametrize("ctx", [5, 84, 84 + 63, 84 + 64, 700])
def test_paged_q_prefill_and_decode(bits, group, ctx):
    n_sink, window, batch = 4, 16, 3
    mask = mask_with_counts(np.random.default_rng(ctx + group + bits), COUNTS)
    n_kv = mask.shape[0]
    cache = make_paged_q(mask, batch, n_kv * group, n_sink, window, 720, bits, seed=ctx)
    gen = torch.Generator(device=DEV).manual_seed(ctx * 7 + group + bits)
    k = random_bf16((batch, n_kv, ctx, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, ctx, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    case("paged quant prefill", bits, group, ctx)
    dac.leank_pack_k(cache, k, v)
    out = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    assert_quant_cache_matches(cache, bf16_bits(k), bf16_bits(v), mask)
    unused_pages_untouched(cache)
    assert_close(out.cpu().numpy(), _oracle_q(q, k, v, mask, n_sink, window, bits),
                 f"paged quant bits {bits} G {group} ctx {ctx}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n_sink,window", [(4, 16), (6, 0)])
def test_paged_q_appends_and_steps(bits, n_sink, window):
    """Single-token appends, chunked appends and fused steps across group
    (page) completions."""
    batch, group, t0 = 2, 4, n_sink + window + 40
    chunks = [1, 30, 64, 3]
    steps = 70
    total = t0 + sum(chunks) + steps
    mask = mask_with_counts(np.random.default_rng(bits + window), COUNTS)
    n_kv = mask.shape[0]
    cache = make_paged_q(mask, batch, n_kv * group, n_sink, window, total, bits, seed=bits * 3 + window)
    gen = torch.Generator(device=DEV).manual_seed(bits * 11 + window)
    k = random_bf16((batch, n_kv, total, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, total, 128), gen)
    kh, vh = bf16_bits(k), bf16_bits(v)
    case("paged quant appends", bits, n_sink, window)
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    pos = t0
    for n in chunks:
        dac.leank_pack_k(cache, k[:, :, pos:pos + n].contiguous(), v[:, :, pos:pos + n].contiguous(),
                         pos0=pos)
        pos += n
    torch.cuda.synchronize()
    assert_quant_cache_matches(cache, kh[:, :, :pos], vh[:, :, :pos], mask)
    for s in range(steps):
        q = random_bf16((batch, n_kv * group, 128), gen)
        out = dac.leank_decode_step(cache, q, k[:, :, pos].contiguous(), v[:, :, pos].contiguous(),
                                    pos=pos)
        pos += 1
        if s in (0, 1, 30, 31, steps - 1) or (pos - n_sink - window) % 64 == 0:
            torch.cuda.synchronize()
            assert_close(out.cpu().numpy(),
                         _oracle_q(q, k[:, :, :pos], v[:, :, :pos], mask, n_sink, window, bits),
                         f"paged quant step {s}")
    torch.cuda.synchronize()
    assert_quant_cache_matches(cache, kh[:, :, :pos], vh[:, :, :pos], mask)
    unused_pages_untouched(cache)


@pytest.mark.parametrize("bits", [4, 8])
def test_paged_q_ragged(bits):
    """Ragged appends, decode and steps on a paged low-bit cache."""
    n_sink, window, group = 4, 16, 2
    lens = [1, 40, 83, 84, 150]
    max_ctx = 260
    mask = mask_with_counts(np.random.default_rng(81 + bits), [32, 0, 64, 8])
    n_kv = mask.shape[0]
    batch = len(lens)
    cache = make_paged_q(mask, batch, n_kv * group, n_sink, window, max_ctx, bits, seed=83 + bits)
    gen = torch.Generator(device=DEV).manual_seed(89 + bits)
    width = max(lens) + 80
    k = random_bf16((batch, n_kv, width, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, width, 128), gen)
    kh, vh = bf16_bits(k), bf16_bits(v)
    case("paged quant ragged", bits)
    n_new = max(lens)
    dac.leank_pack_k_rows(cache, k[:, :, :n_new].contiguous(), v[:, :, :n_new].contiguous(),
                          torch.zeros(batch, dtype=torch.int64, device=DEV),
                          torch.tensor(lens, dtype=torch.int32, device=DEV))
    q = random_bf16((batch, n_kv * group, 128), gen)
    out = dac.leank_decode_attn_rows(cache, q, torch.tensor(lens, dtype=torch.int32, device=DEV),
                                     max_ctx_len=max(lens))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, n in enumerate(lens):
        assert_quant_cache_matches(cache, kh[b:b + 1, :, :n], vh[b:b + 1, :, :n], mask, rows=[b])
        assert_close(got[b:b + 1],
                     _oracle_q(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], mask, n_sink, window, bits),
                     f"paged quant ragged decode row {b}")
    pos = list(lens)
    for s in range(70):
        q = random_bf16((batch, n_kv * group, 128), gen)
        idx = torch.tensor(pos, dtype=torch.int64, device=DEV)
        kn = torch.stack([k[b, :, pos[b]] for b in range(batch)]).contiguous()
        vn = torch.stack([v[b, :, pos[b]] for b in range(batch)]).contiguous()
        out = dac.leank_decode_step_rows(cache, q, kn, vn, idx, max_ctx_len=max_ctx)
        pos = [p + 1 for p in pos]
        if s in (0, 43, 44, 69):
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for b in range(batch):
                n = pos[b]
                assert_close(got[b:b + 1],
                             _oracle_q(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], mask,
                                       n_sink, window, bits), f"paged quant ragged step {s} row {b}")
                assert_quant_cache_matches(cache, kh[b:b + 1, :, :n], vh[b:b + 1, :, :n], mask, rows=[b])
    unused_pages_untouched(cache)


@pytest.mark.parametrize("bits", [4, 8])
def test_full_workload_paged_quant_sampled(bits):
    """The Llama B64 4K cache with its middle in shuffled 64-row pages: two
    fused steps against the oracle on sampled (row, query head) outputs.
    Each wavefront walks several complete groups per item here, so the
    group loop (and, at 4 bits, its page prefetch) runs at full length."""
    from synthetic import alpha_for, get_config, make_kv, make_q

    cfg = get_config("llama_b64_4k")
    om, okc, oki = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
    case("paged quant full workload", bits)
    ppr = -(-(cfg.ctx - cfg.n_sink - cfg.window) // 64)
    n_pages = cfg.batch * ppr + 3
    table = shuffled_block_table(np.random.default_rng(bits + 11), cfg.batch, ppr, n_pages)
    cache = dac.LayerCache(okc[0].tolist(), torch.from_numpy(oki[0]).to(DEV), cfg.batch,
                           cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, cfg.ctx,
                           device=DEV, n_pages=n_pages, block_table=table, quant_bits=bits)
    k, v = make_kv(cfg, 0, device=DEV)
    t0 = cfg.ctx - 2
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    rng = np.random.default_rng(bits + 5)
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
        assert_close(np.stack([got[b, j] for b, j in pairs]), ref, f"paged bits {bits} step {s}")
