"""GPU path (through the C ABI) against the CPU oracle.

Mask and pack are compared bit for bit; attention outputs element by element
within |gpu - oracle| <= 2e-3 + 1e-2 |oracle|.  Every test prints its case
before touching the GPU.
"""

import math

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import CONFIGS, alpha_for, bf16_bits, get_config, make_kv, make_q
from tests.gpu_cases import (
    assert_cache_matches,
    assert_close,
    kept_from_mask,
    make_cache,
    mask_with_counts,
    oracle_outputs,
    random_bf16,
)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(*args):
    print("CASE", *args, flush=True)


# ---------------------------------------------------------------- mask (bit-exact)

@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_build_mask_matches_oracle_on_workloads(cfg):
    case("build_mask", cfg.name)
    alpha = alpha_for(cfg)
    mask, kept_count, kept_idx = dac.leank_build_mask(torch.from_numpy(alpha).to(DEV),
                                                      cfg.prune_pct, cfg.align)
    om, okc, oki = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    assert np.array_equal(mask.cpu().numpy(), om)
    assert np.array_equal(kept_count.cpu().numpy(), okc)
    assert np.array_equal(kept_idx.cpu().numpy(), oki)


def _alpha_cases(rng):
    yield "ties", rng.integers(0, 5, size=(3, 5, 16)).astype(np.float32)
    yield "tie_free", rng.random((2, 8, 128)).astype(np.float32)
    signed = rng.standard_normal((4, 4, 64)).astype(np.float32)
    signed[0, 0, :5] = [np.inf, -np.inf, 0.0, -0.0, 1e-45]
    signed[1, 2, :3] = [-0.0, 0.0, -0.0]
    yield "signed_inf_zero", signed
    yield "one_head", rng.random((1, 1, 8)).astype(np.float32)
    yield "many_layers", np.abs(rng.standard_normal((32, 8, 128))).astype(np.float32)
    yield "wide_head", rng.integers(0, 50, size=(2, 3, 1024)).astype(np.float32)
    yield "all_equal", np.full((2, 2, 32), 0.5, dtype=np.float32)


def test_build_mask_matches_oracle_random():
    rng = np.random.default_rng(101)
    for name, alpha in _alpha_cases(rng):
        d = alpha.shape[2]
        aligns = [a for a in (8, 16, 32, 64) if d % a == 0]
        for p in (0, 1, 33, 50, 70, 80, 99, 100):
            for align in aligns:
                case("build_mask", name, alpha.shape, p, align)
                mask, kept_count, kept_idx = dac.leank_build_mask(
                    torch.from_numpy(alpha).to(DEV), p, align)
                om, okc, oki = oracle.build_mask(alpha, p, align)
                assert np.array_equal(mask.cpu().numpy(), om), (name, p, align)
                assert np.array_equal(kept_count.cpu().numpy(), okc), (name, p, align)
                assert np.array_equal(kept_idx.cpu().numpy(), oki), (name, p, align)
                # the host form gives the same bits from host memory
                hm, hkc, hki = dac.leank_build_mask(torch.from_numpy(alpha), p, align)
                assert np.array_equal(hm.numpy(), om) and np.array_equal(hkc.numpy(), okc)
                assert np.array_equal(hki.numpy(), oki), (name, p, align)


def test_build_mask_refuses_aligns_the_plan_cannot_take():
    """Kept counts must be multiples of 8 for the cache plan: align 1, 2, 4
    are refused at mask time, before any launch."""
    alpha = torch.rand((1, 2, 128), device=DEV)
    for align in (1, 2, 4):
        case("build_mask align", align)
        with pytest.raises(dac.LeankError) as err:
            dac.leank_build_mask(alpha, 50, align)
        assert err.value.status == -2


def test_build_mask_rejects_nan():
    case("build_mask nan")
    alpha = torch.rand((1, 2, 128), device=DEV)
    alpha[0, 1, 7] = float("nan")
    with pytest.raises(dac.LeankError) as err:
        dac.leank_build_mask(alpha, 50, 32)
    assert err.value.status == -1


# ---------------------------------------------------------------- pack (bit-exact)

PACK_COUNTS = [32, 0, 8, 128, 24, 64]


@pytest.mark.parametrize("n_sink,window", [(4, 16), (0, 8), (3, 1), (5, 0)])
@pytest.mark.parametrize("ctx", [1, 3, 4, 19, 20, 21, 100, 333])
def test_bulk_pack_matches_oracle(n_sink, window, ctx):
    if n_sink + window == 0:
        pytest.skip("no full-width region")
    case("pack bulk", n_sink, window, ctx)
    rng = np.random.default_rng(ctx * 31 + window)
    mask = mask_with_counts(rng, PACK_COUNTS)
    batch = 3
    cache = make_cache(mask, batch, 2 * len(PACK_COUNTS), n_sink, window, max_ctx=400)
    gen = torch.Generator(device=DEV).manual_seed(ctx)
    k = random_bf16((batch, len(PACK_COUNTS), ctx, 128), gen)
    v = random_bf16((batch, len(PACK_COUNTS), ctx, 128), gen)
    dac.leank_pack_k(cache, k, v)
    torch.cuda.synchronize()
    assert cache.length == ctx
    assert_cache_matches(cache, bf16_bits(k), bf16_bits(v), mask)


@pytest.mark.parametrize("chunks", ["ones", "mixed", "wide"])
def test_sequential_appends_match_bulk(chunks):
    n_sink, window, ctx = 4, 16, 230
    rng = np.random.default_rng(7)
    mask = mask_with_counts(rng, PACK_COUNTS)
    batch = 2
    gen = torch.Generator(device=DEV).manual_seed(99)
    k = random_bf16((batch, len(PACK_COUNTS), ctx, 128), gen)
    v = random_bf16((batch, len(PACK_COUNTS), ctx, 128), gen)
    cache = make_cache(mask, batch, len(PACK_COUNTS), n_sink, window, max_ctx=ctx)
    if chunks == "ones":
        sizes = [1] * ctx
    elif chunks == "mixed":
        sizes = []
        while sum(sizes) < ctx:
            sizes.append(int(rng.choice([1, 2, 3, window - 1, window, window + 1, 2 * window + 5])))
    else:
        sizes = [17, 33, 64, 1, 15, 100]
    pos = 0
    for n in sizes:
        n = min(n, ctx - pos)
        if n == 0:
            break
        case("pack sequential", chunks, pos, n)
        dac.leank_pack_k(cache, k[:, :, pos:pos + n].contiguous(), v[:, :, pos:pos + n].contiguous())
        pos += n
        if pos in (1, 4, 19, 20, 21, 50) or pos == ctx:
            torch.cuda.synchronize()
            assert_cache_matches(cache, bf16_bits(k[:, :, :pos]), bf16_bits(v[:, :, :pos]), mask)
    assert pos == ctx


def test_pack_capacity_error():
    case("pack capacity")
    mask = mask_with_counts(np.random.default_rng(1), [32, 0])
    cache = make_cache(mask, 1, 2, 2, 4, max_ctx=10)
    k = torch.zeros((1, 2, 11, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dac.LeankError) as err:
        dac.leank_pack_k(cache, k, k)
    assert err.value.status == -3


# ---------------------------------------------------------------- decode

def _decode_case(mask, batch, group, n_sink, window, ctx, seed, k_scale=1.0, pairs=None):
    n_kv = mask.shape[0]
    cache = make_cache(mask, batch, n_kv * group, n_sink, window, max_ctx=ctx + 3)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    k = random_bf16((batch, n_kv, ctx, 128), gen, scale=k_scale)
    v = random_bf16((batch, n_kv, ctx, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    dac.leank_pack_k(cache, k, v)
    out = torch.full((batch, n_kv * group, 128), float("nan"), device=DEV)
    dac.leank_decode_attn(cache, q, out=out)
    torch.cuda.synchronize()
    ref = oracle_outputs(q, k, v, mask, n_sink, window, pairs=pairs)
    got = out.cpu().numpy()
    if pairs is not None:
        got = np.stack([got[b, j] for b, j in pairs])
    return got, ref


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_every_group_size(group):
    counts = [32, 0, 64, 128, 8, 16, 24, 96]
    rng = np.random.default_rng(group)
    mask = mask_with_counts(rng, counts)
    for ctx in (1, 37, 700):
        case("decode group", group, ctx)
        got, ref = _decode_case(mask, 2, group, 8, 32, ctx, seed=group * 100 + ctx, k_scale=2.0)
        assert_close(got, ref, f"group={group} ctx={ctx}")


@pytest.mark.parametrize("kept", [8, 16, 24, 32, 40, 48, 56, 64, 72, 80, 88, 96, 104, 112, 120, 128])
def test_decode_every_kept_width(kept):
    rng = np.random.default_rng(kept)
    mask = mask_with_counts(rng, [kept, 0, kept])
    case("decode width", kept)
    got, ref = _decode_case(mask, 3, 4, 4, 64, 1500, seed=kept, k_scale=2.0)
    assert_close(got, ref, f"kept={kept}")


@pytest.mark.parametrize("ctx", [1, 2, 63, 64, 65, 127, 128, 129, 576, 577, 1000, 4097])
def test_decode_region_boundaries(ctx):
    rng = np.random.default_rng(ctx)
    mask = mask_with_counts(rng, [32, 0, 64, 128])
    case("decode boundary", ctx)
    got, ref = _decode_case(mask, 2, 4, 64, 64, ctx, seed=ctx)
    assert_close(got, ref, f"ctx={ctx}")


def test_decode_no_pruning_and_all_dead():
    for counts in ([128, 128], [0, 0]):
        case("decode extremes", counts)
        mask = mask_with_counts(np.random.default_rng(3), counts)
        got, ref = _decode_case(mask, 4, 4, 16, 100, 2000, seed=11)
        assert_close(got, ref, str(counts))


@pytest.mark.parametrize("ctx", [4_000, 7_000, 12_000, 25_000, 50_000, 100_000, 200_000, 340_000])
def test_decode_many_items_per_pair(ctx):
    # one long batch row: its live pair's record count grows from about 17
    # (the one-wavefront combine's two-row form) to over a thousand, so the
    # workgroup combine runs with every channel slice count (1 to 32 slices
    # of the 128 channels)
    mask = mask_with_counts(np.random.default_rng(ctx), [128, 0])
    case("decode many items", ctx)
    got, ref = _decode_case(mask, 1, 4, 64, 512, ctx, seed=ctx)
    assert_close(got, ref, f"ctx={ctx}")


def test_decode_large_scores():
    # large K spreads the softmax over few tokens: exercises the running max
    mask = mask_with_counts(np.random.default_rng(5), [32, 64, 0, 128])
    case("decode large scores")
    got, ref = _decode_case(mask, 2, 2, 4, 32, 3000, seed=5, k_scale=12.0)
    assert_close(got, ref, "large scores")


def test_tiny_workload_end_to_end():
    cfg = get_config("tiny")
    case("tiny end to end")
    alpha = alpha_for(cfg)
    mask, kept_count, kept_idx = dac.leank_build_mask(torch.from_numpy(alpha).to(DEV),
                                                      cfg.prune_pct, cfg.align)
    cache = dac.LayerCache(kept_count[0].cpu().tolist(), kept_idx[0].contiguous(), cfg.batch,
                           cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, cfg.ctx)
    k, v = make_kv(cfg, 0, device=DEV)
    q = make_q(cfg, 0, device=DEV)
    dac.leank_pack_k(cache, k, v)
    out = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    om, _, _ = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    assert_cache_matches(cache, bf16_bits(k), bf16_bits(v), om[0])
    ref = oracle_outputs(q, k, v, om[0], cfg.n_sink, cfg.window)
    assert_close(out.cpu().numpy(), ref, "tiny")


def test_workspace_reuse_across_context_lengths():
    mask = mask_with_counts(np.random.default_rng(8), [32, 0, 64, 16])
    n_sink, window, batch, group = 4, 40, 2, 2
    ctx_max = 900
    cache = make_cache(mask, batch, 4 * group, n_sink, window, max_ctx=ctx_max)
    gen = torch.Generator(device=DEV).manual_seed(8)
    k = random_bf16((batch, 4, ctx_max, 128), gen)
    v = random_bf16((batch, 4, ctx_max, 128), gen)
    q = random_bf16((batch, 4 * group, 128), gen)
    ws = torch.full((dac.leank_workspace_bytes(cache, ctx_max),), 0xAB, dtype=torch.uint8, device=DEV)
    dac.leank_workspace_init(ws)
    pos = 0
    for ctx in (5, 44, 45, 300, 301, 899, 900):
        case("workspace reuse", ctx)
        dac.leank_pack_k(cache, k[:, :, pos:ctx].contiguous(), v[:, :, pos:ctx].contiguous())
        pos = ctx
        for _ in range(2):
            out = dac.leank_decode_attn(cache, q, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle_outputs(q, k[:, :, :ctx], v[:, :, :ctx], mask, n_sink, window)
        assert_close(out.cpu().numpy(), ref, f"ctx={ctx}")


# ---------------------------------------------------------------- full-size workloads, sampled

def _sample_pairs(cfg, rng, n_random):
    pairs = {(0, j) for j in range(cfg.n_q_heads)} | {(cfg.batch - 1, j) for j in range(cfg.n_q_heads)}
    for _ in range(n_random):
        pairs.add((int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_q_heads))))
    return sorted(pairs)


@pytest.mark.parametrize("name", ["llama_b64_4k", "qwen_b16_32k"])
def test_full_workload_sampled(name):
    cfg = get_config(name)
    case("full workload", name)
    alpha = alpha_for(cfg)
    mask, kept_count, kept_idx = dac.leank_build_mask(torch.from_numpy(alpha).to(DEV),
                                                      cfg.prune_pct, cfg.align)
    om, _, _ = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    assert np.array_equal(mask.cpu().numpy(), om)
    cache = dac.LayerCache(kept_count[0].cpu().tolist(), kept_idx[0].contiguous(), cfg.batch,
                           cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, cfg.ctx)
    k, v = make_kv(cfg, 0, device=DEV)
    q = make_q(cfg, 0, device=DEV)
    dac.leank_pack_k(cache, k, v)
    out = torch.full(tuple(q.shape), float("nan"), device=DEV)
    dac.leank_decode_attn(cache, q, out=out)
    again = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert torch.equal(out, again), "repeated decode is not bit-identical"
    pairs = _sample_pairs(cfg, np.random.default_rng(cfg.index), 40)
    kh, vh, qh = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    ref = oracle.decode(qh, kh, vh, om[0], cfg.n_sink, cfg.window, pairs=pairs)
    assert_close(np.stack([got[b, j] for b, j in pairs]), ref, name)
    # packed state of the sampled (b, h) pairs
    kv_pairs = sorted({(b, j // cfg.group) for b, j in pairs})[:12]
    sel_k = np.stack([kh[b, h] for b, h in kv_pairs])[:, None]
    sel_v = np.stack([vh[b, h] for b, h in kv_pairs])[:, None]
    assert_cache_matches(cache, sel_k, sel_v, om[0], pairs=kv_pairs)


def test_long_context_all_layers_sampled():
    cfg = get_config("llama32_b1_128k")
    alpha = alpha_for(cfg)
    mask, kept_count, kept_idx = dac.leank_build_mask(torch.from_numpy(alpha).to(DEV),
                                                      cfg.prune_pct, cfg.align)
    om, okc, _ = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    assert np.array_equal(mask.cpu().numpy(), om)
    rng = np.random.default_rng(3)
    for layer in range(cfg.n_layers):
        case("long context layer", layer)
        cache = dac.LayerCache(kept_count[layer].cpu().tolist(), kept_idx[layer].contiguous(),
                               cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window,
                               cfg.ctx)
        k, v = make_kv(cfg, layer, device=DEV)
        q = make_q(cfg, layer, device=DEV)
        dac.leank_pack_k(cache, k, v)
        out = dac.leank_decode_attn(cache, q)
        torch.cuda.synchronize()
        live = [h for h in range(cfg.n_kv_heads) if okc[layer, h] > 0]
        dead = [h for h in range(cfg.n_kv_heads) if okc[layer, h] == 0]
        heads = []
        if live:
            heads.append(live[int(rng.integers(len(live)))])
        if dead and layer % 4 == 0:
            heads.append(dead[int(rng.integers(len(dead)))])
        pairs = [(0, h * cfg.group + g) for h in heads for g in range(cfg.group)]
        kh = bf16_bits(k[:, heads])
        vh = bf16_bits(v[:, heads])
        # oracle on the selected heads only (same query heads, one KV head each)
        for n, h in enumerate(heads):
            qsel = bf16_bits(q[:, h * cfg.group:(h + 1) * cfg.group])
            ref = oracle.decode(qsel, kh[:, n:n + 1], vh[:, n:n + 1], om[layer][h:h + 1],
                                cfg.n_sink, cfg.window)
            got = out[:, h * cfg.group:(h + 1) * cfg.group].cpu().numpy()
            assert_close(got, ref, f"layer {layer} head {h}")
        del cache, k, v
        torch.cuda.empty_cache()
    assert math.isfinite(float(out.abs().max()))
