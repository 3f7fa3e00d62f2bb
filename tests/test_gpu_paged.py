"""Paged middle (64-row pages from a pool through a block table) against
the CPU oracle: cache rows read back through the table bit for bit,
attention within 2e-3 + 1e-2 |oracle|, pages outside the table untouched."""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import (assert_cache_matches, assert_close, kept_from_mask, mask_with_counts,
                             random_bf16, shuffled_block_table)

pytestmark = pytest.mark.gpu
DEV = "cuda"
COUNTS = [32, 0, 64, 128, 8]
SENTINEL = 0x7FC1  # a bf16 NaN pattern: any read of a page outside the table shows up


def case(*args):
    print("CASE", *args, flush=True)


def make_paged(mask, batch, n_q, n_sink, window, max_ctx, seed, spare=5):
    kept_count, kept_idx = kept_from_mask(mask)
    mid_cap = max(0, max_ctx - n_sink - window)
    ppr = -(-mid_cap // 64)
    n_pages = batch * ppr + spare
    table = shuffled_block_table(np.random.default_rng(seed), batch, ppr, n_pages)
    cache = dac.LayerCache(kept_count.tolist(), torch.from_numpy(kept_idx).to(DEV), batch, n_q,
                           mask.shape[0], n_sink, window, max_ctx, device=DEV, n_pages=n_pages,
                           block_table=table)
    cache.pool.view(torch.int16).fill_(SENTINEL)
    return cache


def unused_pages_untouched(cache):
    used = set(cache.block_table.cpu().numpy().ravel().tolist())
    pe = cache.desc.page_bytes // 2
    pool = bf16_bits(cache.pool)
    for page in range(cache.desc.n_pages):
        if page not in used:
            assert np.all(pool[page * pe:(page + 1) * pe] == SENTINEL), page


@pytest.mark.parametrize("group", [1, 4, 7])
@pytest.mark.parametrize("ctx", [5, 84, 84 + 63, 84 + 64, 1000])
def test_paged_prefill_and_decode(group, ctx):
    n_sink, window, batch = 4, 16, 3
    mask = mask_with_counts(np.random.default_rng(ctx + group), COUNTS)
    n_kv = mask.shape[0]
    cache = make_paged(mask, batch, n_kv * group, n_sink, window, 1024, seed=ctx)
    gen = torch.Generator(device=DEV).manual_seed(ctx * 7 + group)
    k = random_bf16((batch, n_kv, ctx, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, ctx, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    case("paged prefill", group, ctx)
    dac.leank_pack_k(cache, k, v)
    out = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    kh, vh = bf16_bits(k), bf16_bits(v)
    assert_cache_matches(cache, kh, vh, mask)
    assert_close(out.cpu().numpy(), oracle.decode(bf16_bits(q), kh, vh, mask, n_sink, window),
                 f"paged G {group} ctx {ctx}")
    unused_pages_untouched(cache)


@pytest.mark.parametrize("window", [16, 0])
def test_paged_fused_steps_across_pages(window):
    n_sink, batch, group = 4, 2, 4
    t0, steps = n_sink + window + 60, 140
    mask = mask_with_counts(np.random.default_rng(window), COUNTS)
    n_kv = mask.shape[0]
    cache = make_paged(mask, batch, n_kv * group, n_sink, window, t0 + steps, seed=3 + window)
    gen = torch.Generator(device=DEV).manual_seed(window + 1)
    k = random_bf16((batch, n_kv, t0 + steps, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, t0 + steps, 128), gen)
    q = random_bf16((steps, batch, n_kv * group, 128), gen)
    case("paged steps", window)
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    outs = [dac.leank_decode_step(cache, q[s], k[:, :, t0 + s].contiguous(),
                                  v[:, :, t0 + s].contiguous()) for s in range(steps)]
    torch.cuda.synchronize()
    kh, vh, qh = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    assert_cache_matches(cache, kh, vh, mask)
    for s in range(0, steps, 7):
        ref = oracle.decode(qh[s], kh[:, :, :t0 + s + 1], vh[:, :, :t0 + s + 1], mask, n_sink, window)
        assert_close(outs[s].cpu().numpy(), ref, f"paged step {s}")
    unused_pages_untouched(cache)


def test_paged_ragged_rows():
    n_sink, window, group, max_ctx = 4, 16, 2, 500
    lengths = [0, 3, 20, 21, 84, 85, 300, 400]
    batch = len(lengths)
    mask = mask_with_counts(np.random.default_rng(12), COUNTS)
    n_kv = mask.shape[0]
    cache = make_paged(mask, batch, n_kv * group, n_sink, window, max_ctx, seed=12)
    gen = torch.Generator(device=DEV).manual_seed(12)
    k = random_bf16((batch, n_kv, max_ctx, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, max_ctx, 128), gen)
    steps = 20
    q = random_bf16((steps, batch, n_kv * group, 128), gen)
    case("paged ragged")
    n_pre = max(lengths)
    dac.leank_pack_k_rows(cache, k[:, :, :n_pre].contiguous(), v[:, :, :n_pre].contiguous(),
                          torch.zeros(batch, dtype=torch.int64, device=DEV),
                          torch.tensor(lengths, dtype=torch.int32, device=DEV))
    lens = list(lengths)
    kh, vh, qh = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    for s in range(steps):
        kk = torch.stack([k[b, :, lens[b]] for b in range(batch)]).contiguous()
        vv = torch.stack([v[b, :, lens[b]] for b in range(batch)]).contiguous()
        out = dac.leank_decode_step_rows(cache, q[s], kk, vv,
                                         torch.tensor(lens, dtype=torch.int64, device=DEV),
                                         max_ctx_len=max(lens) + 1)
        lens = [n + 1 for n in lens]
        if s % 6 == 5:
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for b in range(batch):
                ref = oracle.decode(qh[s, b:b + 1], kh[b:b + 1, :, :lens[b]], vh[b:b + 1, :, :lens[b]],
                                    mask, n_sink, window)
                assert_close(got[b:b + 1], ref, f"paged ragged step {s} row {b}")
    torch.cuda.synchronize()
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = dac.leank_decode_attn_rows(cache, q[0], ctx, max_ctx_len=max(lens))
    torch.cuda.synchronize()
    for b in range(batch):
        pairs = [(b, h) for h in range(n_kv)]
        sel_k = np.stack([kh[b, h, :lens[b]] for h in range(n_kv)])[:, None]
        sel_v = np.stack([vh[b, h, :lens[b]] for h in range(n_kv)])[:, None]
        assert_cache_matches(cache, sel_k, sel_v, mask, pairs=pairs)
        ref = oracle.decode(qh[0, b:b + 1], kh[b:b + 1, :, :lens[b]], vh[b:b + 1, :, :lens[b]], mask,
                            n_sink, window)
        assert_close(out.cpu().numpy()[b:b + 1], ref, f"paged ragged decode row {b}")


def test_paged_full_workload_sampled():
    from synthetic import alpha_for, get_config, make_kv, make_q

    cfg = get_config("llama_b64_4k")
    om, okc, oki = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
    case("paged full workload")
    ppr = -(-(cfg.ctx - cfg.n_sink - cfg.window) // 64)
    n_pages = cfg.batch * ppr + 3
    table = shuffled_block_table(np.random.default_rng(5), cfg.batch, ppr, n_pages)
    cache = dac.LayerCache(okc[0].tolist(), torch.from_numpy(oki[0]).to(DEV), cfg.batch,
                           cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, cfg.ctx,
                           n_pages=n_pages, block_table=table)
    k, v = make_kv(cfg, 0, device=DEV)
    t0 = cfg.ctx - 2
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    rng = np.random.default_rng(6)
    pairs = sorted({(int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_q_heads)))
                    for _ in range(16)} | {(0, 0), (cfg.batch - 1, cfg.n_q_heads - 1)})
    kh, vh = bf16_bits(k), bf16_bits(v)
    for s in range(2):
        q = make_q(cfg, 0, step=s + 1, device=DEV)
        out = dac.leank_decode_step(cache, q, k[:, :, t0 + s].contiguous(), v[:, :, t0 + s].contiguous())
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = oracle.decode(bf16_bits(q), kh[:, :, :t0 + s + 1], vh[:, :, :t0 + s + 1], om[0],
                            cfg.n_sink, cfg.window, pairs=pairs)
        assert_close(np.stack([got[b, j] for b, j in pairs]), ref, f"paged llama step {s}")
    kv_pairs = sorted({(b, j // cfg.group) for b, j in pairs})[:8]
    assert_cache_matches(cache, np.stack([kh[b, h] for b, h in kv_pairs])[:, None],
                         np.stack([vh[b, h] for b, h in kv_pairs])[:, None], om[0], pairs=kv_pairs)
