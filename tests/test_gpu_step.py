"""Fused decode step (append one token + attend, in the decode kernels)
against the CPU oracle: the cache after every step is compared bit for bit
with the oracle's packing of all tokens so far, and the output with the
oracle's attention over them, within 2e-3 + 1e-2 |oracle|."""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import alpha_for, bf16_bits, get_config, make_kv, make_q
from tests.gpu_cases import (assert_cache_matches, assert_close, make_cache, mask_with_counts,
                             random_bf16)

pytestmark = pytest.mark.gpu
DEV = "cuda"
COUNTS = [32, 0, 64, 128, 8]


def case(*args):
    print("CASE", *args, flush=True)


@pytest.mark.parametrize("n_sink,window,group", [(4, 16, 3), (0, 16, 4), (3, 5, 1), (4, 1, 8),
                                                 (6, 0, 2), (5, 37, 7)])
def test_steps_from_empty_cache(n_sink, window, group):
    """Every position from 0: sink rows, ring filling, ring wrap, middle rows."""
    batch, steps = 3, 120
    mask = mask_with_counts(np.random.default_rng(10 + window), COUNTS)
    n_kv = mask.shape[0]
    cache = make_cache(mask, batch, n_kv * group, n_sink, window, steps + 7)
    gen = torch.Generator(device=DEV).manual_seed(100 + n_sink * 31 + window)
    k = random_bf16((batch, n_kv, steps, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, steps, 128), gen)
    q = random_bf16((steps, batch, n_kv * group, 128), gen)
    kh, vh, qh = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    case("steps from empty", n_sink, window, group)
    outs = []
    for pos in range(steps):
        out = dac.leank_decode_step(cache, q[pos], k[:, :, pos].contiguous(),
                                    v[:, :, pos].contiguous())
        outs.append(out)
        if pos % 17 == 0 or pos in (n_sink, n_sink + window, n_sink + window + 1):
            torch.cuda.synchronize()
            assert_cache_matches(cache, kh[:, :, :pos + 1], vh[:, :, :pos + 1], mask)
    assert cache.length == steps
    torch.cuda.synchronize()
    assert_cache_matches(cache, kh, vh, mask)
    for pos in range(steps):
        ref = oracle.decode(qh[pos], kh[:, :, :pos + 1], vh[:, :, :pos + 1], mask, n_sink, window)
        assert_close(outs[pos].cpu().numpy(), ref, f"pos {pos}")


@pytest.mark.parametrize("group", [1, 4, 7, 8])
def test_steps_after_prefill(group):
    """Bulk prefill over several tiles, then steps; fused and unfused agree."""
    n_sink, window, batch, t0, steps = 4, 64, 2, 1000, 40
    mask = mask_with_counts(np.random.default_rng(group), COUNTS)
    n_kv = mask.shape[0]
    fused = make_cache(mask, batch, n_kv * group, n_sink, window, t0 + steps)
    plain = make_cache(mask, batch, n_kv * group, n_sink, window, t0 + steps)
    gen = torch.Generator(device=DEV).manual_seed(group)
    k = random_bf16((batch, n_kv, t0 + steps, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, t0 + steps, 128), gen)
    q = random_bf16((steps, batch, n_kv * group, 128), gen)
    case("steps after prefill", group)
    for cache in (fused, plain):
        dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    outs, plain_outs = [], []
    for s in range(steps):
        kk, vv = k[:, :, t0 + s].contiguous(), v[:, :, t0 + s].contiguous()
        outs.append(dac.leank_decode_step(fused, q[s], kk, vv))
        dac.leank_pack_k(plain, kk[:, :, None], vv[:, :, None])
        plain_outs.append(dac.leank_decode_attn(plain, q[s]))
    torch.cuda.synchronize()
    kh, vh, qh = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    assert_cache_matches(fused, kh, vh, mask)
    assert_cache_matches(plain, kh, vh, mask)
    for s in range(steps):
        ref = oracle.decode(qh[s], kh[:, :, :t0 + s + 1], vh[:, :, :t0 + s + 1], mask, n_sink,
                            window)
        assert_close(outs[s].cpu().numpy(), ref, f"fused step {s}")
        assert_close(plain_outs[s].cpu().numpy(), ref, f"unfused step {s}")


def test_step_rows_ragged():
    """Per-row positions, rows left out by an out-of-range position."""
    n_sink, window, group, max_ctx = 4, 16, 2, 400
    lengths = [0, 3, 4, 19, 20, 21, 300, 350]
    batch = len(lengths)
    mask = mask_with_counts(np.random.default_rng(77), COUNTS)
    n_kv = mask.shape[0]
    cache = make_cache(mask, batch, n_kv * group, n_sink, window, max_ctx)
    gen = torch.Generator(device=DEV).manual_seed(77)
    k = random_bf16((batch, n_kv, max_ctx, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, max_ctx, 128), gen)
    steps = 30
    q = random_bf16((steps, batch, n_kv * group, 128), gen)
    kh, vh, qh = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    case("step rows prefill")
    n_pre = max(lengths)
    dac.leank_pack_k_rows(cache, k[:, :, :n_pre].contiguous(), v[:, :, :n_pre].contiguous(),
                          torch.zeros(batch, dtype=torch.int64, device=DEV),
                          torch.tensor(lengths, dtype=torch.int32, device=DEV))
    lens = list(lengths)
    rng = np.random.default_rng(3)
    for s in range(steps):
        # most rows append, some sit out through a position the call ignores
        skip = [bool(rng.random() < 0.2) for _ in range(batch)]
        pos = [(-1 if b % 2 else 10 ** 6) if skip[b] else lens[b] for b in range(batch)]
        bound = max(lens) + 1
        kk = torch.stack([k[b, :, min(lens[b], max_ctx - 1)] for b in range(batch)]).contiguous()
        vv = torch.stack([v[b, :, min(lens[b], max_ctx - 1)] for b in range(batch)]).contiguous()
        case("step rows", s, pos)
        out = dac.leank_decode_step_rows(cache, q[s], kk, vv,
                                         torch.tensor(pos, dtype=torch.int64, device=DEV),
                                         max_ctx_len=bound)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for b in range(batch):
            if skip[b]:
                assert np.all(got[b] == 0.0), (s, b)
                continue
            lens[b] += 1
            ref = oracle.decode(qh[s, b:b + 1], kh[b:b + 1, :, :lens[b]], vh[b:b + 1, :, :lens[b]],
                                mask, n_sink, window)
            assert_close(got[b:b + 1], ref, f"step {s} row {b}")
        if s % 10 == 9:
            for b in range(batch):
                pairs = [(b, h) for h in range(n_kv)]
                if lens[b] == 0:
                    continue
                sel_k = np.stack([kh[b, h, :lens[b]] for h in range(n_kv)])[:, None]
                sel_v = np.stack([vh[b, h, :lens[b]] for h in range(n_kv)])[:, None]
                assert_cache_matches(cache, sel_k, sel_v, mask, pairs=pairs)


def test_step_capacity_and_workspace_errors():
    mask = mask_with_counts(np.random.default_rng(1), [32, 0])
    cache = make_cache(mask, 1, 4, 4, 8, 20)
    gen = torch.Generator(device=DEV).manual_seed(1)
    q = random_bf16((1, 4, 128), gen)
    k = random_bf16((1, 2, 20, 128), gen)
    v = random_bf16((1, 2, 20, 128), gen)
    case("step errors")
    dac.leank_pack_k(cache, k[:, :, :19].contiguous(), v[:, :, :19].contiguous())
    tok_k, tok_v = k[:, :, 19].contiguous(), v[:, :, 19].contiguous()
    with pytest.raises(dac.LeankError) as err:
        dac.leank_decode_step(cache, q, tok_k, tok_v, pos=20)
    assert err.value.status == dac._lib.ECAPACITY
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(dac.LeankError) as err:
        dac.leank_decode_step(cache, q, tok_k, tok_v, pos=19, workspace=small)
    assert err.value.status == dac._lib.EWORKSPACE
    ws = torch.zeros(dac.leank_workspace_bytes(cache, 20), dtype=torch.uint8, device=DEV)
    out = dac.leank_decode_step(cache, q, tok_k, tok_v, pos=19, workspace=ws)  # last row fits
    torch.cuda.synchronize()
    assert cache.length == 20
    ref = oracle.decode(bf16_bits(q), bf16_bits(k), bf16_bits(v), mask, 4, 8)
    assert_close(out.cpu().numpy(), ref, "last position")
    assert_cache_matches(cache, bf16_bits(k), bf16_bits(v), mask)


@pytest.mark.parametrize("name", ["llama_b64_4k", "qwen_b16_32k"])
def test_full_workload_steps_sampled(name):
    """The benchmark's shapes: prefill ctx - 3 tokens, then 3 fused steps."""
    cfg = get_config(name)
    alpha = alpha_for(cfg)
    om, okc, oki = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    case("full workload steps", name)
    cache = dac.LayerCache(okc[0].tolist(), torch.from_numpy(oki[0]).to(DEV), cfg.batch,
                           cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, cfg.ctx)
    k, v = make_kv(cfg, 0, device=DEV)
    t0 = cfg.ctx - 3
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    rng = np.random.default_rng(cfg.index)
    pairs = sorted({(int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_q_heads)))
                    for _ in range(24)} | {(0, 0), (cfg.batch - 1, cfg.n_q_heads - 1)})
    kh, vh = bf16_bits(k), bf16_bits(v)
    for s in range(3):
        q = make_q(cfg, 0, step=s + 1, device=DEV)
        out = dac.leank_decode_step(cache, q, k[:, :, t0 + s].contiguous(),
                                    v[:, :, t0 + s].contiguous())
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got))
        ref = oracle.decode(bf16_bits(q), kh[:, :, :t0 + s + 1], vh[:, :, :t0 + s + 1], om[0],
                            cfg.n_sink, cfg.window, pairs=pairs)
        assert_close(np.stack([got[b, j] for b, j in pairs]), ref, f"{name} step {s}")
    kv_pairs = sorted({(b, j // cfg.group) for b, j in pairs})[:10]
    sel_k = np.stack([kh[b, h] for b, h in kv_pairs])[:, None]
    sel_v = np.stack([vh[b, h] for b, h in kv_pairs])[:, None]
    assert_cache_matches(cache, sel_k, sel_v, om[0], pairs=kv_pairs)


@pytest.mark.parametrize("layout", ["bf16", "paged", "q4", "q8", "paged-q4"])
def test_step_rewrites_shared_v_blocks_unchanged(layout):
    """The step item writes back whole 8-row V blocks (4-bit: code bytes
    that two rows share) while the last middle item reads the same block.
    From a new middle row 3 into its block, across the next block edge, every
    row of every pair stays bit-exact after every step, and the outputs
    match the oracle."""
    from tests.gpu_cases import assert_quant_cache_matches, shuffled_block_table

    n_sink, window, batch, group = 8, 40, 4, 4
    counts = [32, 0, 64, 128]
    bits = 4 if "q4" in layout else 8 if "q8" in layout else 0
    paged = layout.startswith("paged")
    t0 = n_sink + window + 64 * 3 + 3   # the first step moves middle row 195 = 8 * 24 + 3
    steps = 12
    mask = mask_with_counts(np.random.default_rng(77), counts)
    n_kv = len(counts)
    max_ctx = t0 + steps + 1
    kept_count = mask.sum(axis=1).astype(np.int32)
    kept_idx = np.full((n_kv, 128), -1, dtype=np.int16)
    for h in range(n_kv):
        kept_idx[h, :kept_count[h]] = np.flatnonzero(mask[h])
    extra = {}
    if paged:
        ppr = -(-(max_ctx - n_sink - window) // 64)
        n_pages = batch * ppr + 2
        extra = dict(n_pages=n_pages,
                     block_table=shuffled_block_table(np.random.default_rng(5), batch, ppr, n_pages))
    cache = dac.LayerCache(kept_count.tolist(), torch.from_numpy(kept_idx).to(DEV), batch,
                           n_kv * group, n_kv, n_sink, window, max_ctx, device=DEV,
                           quant_bits=bits, **extra)
    gen = torch.Generator(device=DEV).manual_seed(78)
    k = random_bf16((batch, n_kv, t0 + steps, 128), gen, scale=2.0)
    v = random_bf16((batch, n_kv, t0 + steps, 128), gen)
    q = random_bf16((steps, batch, n_kv * group, 128), gen)
    kh, vh = bf16_bits(k), bf16_bits(v)
    case("shared V blocks", layout)
    dac.leank_pack_k(cache, k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous())
    for s in range(steps):
        pos = t0 + s
        out = dac.leank_decode_step(cache, q[s], k[:, :, pos].contiguous(), v[:, :, pos].contiguous())
        torch.cuda.synchronize()
        if bits:
            assert_quant_cache_matches(cache, kh[:, :, :pos + 1], vh[:, :, :pos + 1], mask)
            ref = oracle.decode_q(bf16_bits(q[s]), kh[:, :, :pos + 1], vh[:, :, :pos + 1], mask,
                                  n_sink, window, bits)
        else:
            assert_cache_matches(cache, kh[:, :, :pos + 1], vh[:, :, :pos + 1], mask)
            ref = oracle.decode(bf16_bits(q[s]), kh[:, :, :pos + 1], vh[:, :, :pos + 1], mask,
                                n_sink, window)
        assert_close(out.cpu().numpy(), ref, f"{layout} step {s}")
