"""Seeded random layers against the CPU oracle, across every cache kind.

Each case draws a layer shape (query heads per KV head 1..8, 1..12 KV heads
with kept widths from 0 to 128 in steps of 8, sink and window sizes, batch,
context length; a second set takes 9 to 64 KV heads) and a cache kind
(bf16, paged bf16, 4- and 8-bit middles, paged 4-bit), prefills it, and
checks a decode call or a fused step over sampled (batch row, query head)
pairs against the oracle's attention (`oracle.decode`, or `oracle.decode_q`
over the low-bit streams) within the parity bound; a decode call repeated
gives the same bits.  The draws reach plans the fixed cases may not: one
round or several, balanced rounds, tail items, full-width items first, wide
and narrow heads side by side.
"""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import KINDS, assert_close, build_kind, mask_with_counts, random_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 40


def draw(i):
    rng = np.random.default_rng(20261203 + i)
    group = int(rng.integers(1, 9))
    n_kv = int(rng.choice([1, 2, 3, 4, 8, 12]))
    counts = [int(c) for c in rng.choice([0, 8, 16, 24, 32, 48, 64, 96, 128], size=n_kv)]
    if not any(counts):
        counts[int(rng.integers(n_kv))] = 32
    n_sink = int(rng.choice([0, 4, 64]))
    window = int(rng.choice([1, 16, 512]))
    batch = int(rng.choice([1, 2, 3, 5]))
    kind = KINDS[i % len(KINDS)]
    step = bool(i % 2)
    # at least a few middle pages for the paged kinds; about 200K cached rows
    # at most, 1.5M in every fourth case (plans of more than one round)
    lo = n_sink + window + 130
    rows = 1_500_000 if i % 4 == 3 else 200_000
    hi = max(lo + 1, min(40000 if i % 4 == 3 else 6000, rows // (batch * n_kv)))
    ctx = int(rng.integers(lo, hi))
    return dict(group=group, counts=counts, n_sink=n_sink, window=window, batch=batch, ctx=ctx,
                kind=kind, step=step, seed=20261203 + i)


def draw_wide(i):
    """Layers of 9 to 64 KV heads (the items walk the heads' records) with 1
    to 8 query heads each, at small batches and contexts."""
    rng = np.random.default_rng(20261204 + i)
    group = int(rng.integers(1, 9))
    n_kv = int(rng.integers(9, 65))
    counts = [int(c) for c in rng.choice([0, 8, 16, 24, 32, 48, 64, 96, 128], size=n_kv)]
    if not any(counts):
        counts[int(rng.integers(n_kv))] = 32
    n_sink = int(rng.choice([0, 4, 64]))
    window = int(rng.choice([1, 16, 256]))
    batch = int(rng.choice([1, 2, 3]))
    lo = n_sink + window + 130
    ctx = int(rng.integers(lo, lo + 2500))
    return dict(group=group, counts=counts, n_sink=n_sink, window=window, batch=batch, ctx=ctx,
                kind=KINDS[i % len(KINDS)], step=bool(i % 2), seed=20261204 + i)


N_WIDE = 20


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer(i):
    check(draw(i), f"random case {i}")


@pytest.mark.parametrize("i", range(N_WIDE))
def test_random_wide_layer(i):
    check(draw_wide(i), f"random wide case {i}")


def check(c, what):
    print("CASE", what, c, flush=True)
    rng = np.random.default_rng(c["seed"])
    mask = mask_with_counts(rng, c["counts"])
    n_kv = mask.shape[0]
    n_q = n_kv * c["group"]
    batch, ctx = c["batch"], c["ctx"]
    cache, bits = build_kind(c["kind"], mask, batch, n_q, c["n_sink"], c["window"], ctx + 4, c["seed"])
    gen = torch.Generator(device=DEV).manual_seed(c["seed"])
    k = random_bf16((batch, n_kv, ctx, 128), gen, scale=1.5)
    v = random_bf16((batch, n_kv, ctx, 128), gen)
    q = random_bf16((batch, n_q, 128), gen)
    if c["step"]:
        dac.leank_pack_k(cache, k[:, :, :ctx - 1].contiguous(), v[:, :, :ctx - 1].contiguous())
        out = dac.leank_decode_step(cache, q, k[:, :, ctx - 1].contiguous(), v[:, :, ctx - 1].contiguous())
    else:
        dac.leank_pack_k(cache, k, v)
        out = dac.leank_decode_attn(cache, q)
        # the merge order is fixed: a second call gives the same bits
        again = dac.leank_decode_attn(cache, q)
        torch.cuda.synchronize()
        assert torch.equal(out, again), f"{what}: a repeated decode call differs"
    torch.cuda.synchronize()
    assert cache.length == ctx
    pairs = sorted({(int(rng.integers(batch)), int(rng.integers(n_q))) for _ in range(20)}
                   | {(0, 0), (batch - 1, n_q - 1)})
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    if bits:
        ref = oracle.decode_q(qb, kb, vb, mask, c["n_sink"], c["window"], bits, pairs=pairs)
    else:
        ref = oracle.decode(qb, kb, vb, mask, c["n_sink"], c["window"], pairs=pairs)
    got = out.cpu().numpy()
    assert_close(np.stack([got[b, j] for b, j in pairs]), ref, what)
