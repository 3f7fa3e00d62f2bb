"""Needles at the work plan's boundaries, at full size.

At thousands of tokens a lost or doubled row moves an attention output by
about |v| / T, under the parity bound.  These cases make one row count:
each (batch row, KV head) pair holds N "needle" rows whose keys all give
the same dominant score (about 140 above every other row, so the other rows
weigh less than e^-100 together) and whose values are distinct rows on an
exact grid.  The output of every query head of the pair must then be the
plain mean of the included needles' values: a lost needle, or one counted
twice, moves a channel by up to about 32 / N: over 10x the bound of
2e-3 + 1e-2 |mean| for the few hundred needles per pair of most cases, and
over 5x for the 2000 of the one-live-head case on the 8-bit grid (on the
4-bit grid that case catches a lost or doubled record, which holds several
needles, not a single row).

Needles sit where the kernels split their work: every 64-row quantum of
the middle (item, page and low-bit K-group edges) and the row before it,
32-row tile edges, the first and last middle rows, sink rows, the oldest
and newest window rows and the ring's wrap point, and in a fused step the
appended token and the one it pushes out of the window (whose ring row the
append replaces).  A fully pruned head also holds needles in its middle,
which must have no effect (LeanK page, section 3.2); its output is the mean
of its sink and window needles only (section 3.1 item 2: the region split).

Caches: the Llama-3.1-8B-shaped batch-64 4K layer (its realized mask, one
dead head) and a 128K-token layer at batch 4 with 4 live heads of 64
channels, each as bf16, paged (shuffled block table) and 4- and 8-bit
middles; and a 128K-token layer at batch 1 with one live head, whose
hundreds of items are merged over several channel slices.  A few pairs
are also checked against the CPU oracle.
"""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import assert_close, kept_from_mask, mask_with_counts, random_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
LLAMA_COUNTS = [32, 32, 32, 0, 32, 32, 32, 32]
LONG_COUNTS = [64, 0, 64, 0, 0, 64, 0, 64]
NEEDLE_K = 64.0


def case(*args):
    print("CASE", *args, flush=True)


def special_rows(n_sink, window, ctx, step):
    """Sink, window and step positions of a context of ctx tokens (ctx + 1
    after a step's append)."""
    total = ctx + 1 if step else ctx
    rows = {0, n_sink - 1, total - window, total - 1, n_sink, total - window - 1}
    for p in range(max(n_sink, total - window), total):
        if (p - n_sink) % window in (0, window - 1):
            rows.add(p)
    if step:
        rows |= {ctx, ctx - window}
    return sorted(r for r in rows if 0 <= r < total)


def middle_edges(n_sink, window, total, tiles=True, before=True):
    """Middle positions at 64-row quantum edges (and the row before, when
    `before`), and at 32-row tile edges when `tiles`."""
    lo, hi = n_sink, total - window
    rows = set()
    for m in range(0, hi - lo, 32 if tiles else 64):
        rows.add(lo + m)
        if before:
            rows.add(lo + m - 1)
        if tiles:
            rows.add(lo + m + 1)
    rows |= {lo, hi - 1, hi - 2}
    return sorted(r for r in rows if lo <= r < hi)


def value_levels(rng, bits):
    """Levels of one needle's V row: 0 and the top level both present, so a
    per-token low-bit code holds the row exactly."""
    top = 2 ** bits - 1
    lvl = rng.integers(0, top + 1, size=128)
    a, b = rng.choice(128, size=2, replace=False)
    lvl[a], lvl[b] = 0, top
    return lvl


def to_values(lvl, bits):
    # 4-bit grid -16 + 2 L, 8-bit grid -32 + L/4: multiples of 1/4 below 32
    # in magnitude, exact in bf16; wide, so that one needle in thousands
    # still moves the mean past the bound
    return -16.0 + 2.0 * lvl if bits == 4 else -32.0 + lvl / 4.0


def build_needles(batch, n_q, counts, n_sink, window, ctx, step, bits, seed, per_pair,
                  edges_before=True):
    """K, V [B, H, T, 128] (T = ctx + 1 for a step), q [B, Hq, 128] with
    needles planted, and the expected output [B, Hq, 128] (float64)."""
    rng = np.random.default_rng(seed)
    mask = mask_with_counts(rng, counts)
    n_kv = len(counts)
    group = n_q // n_kv
    total = ctx + 1 if step else ctx
    gen = torch.Generator(device=DEV).manual_seed(seed)
    k = random_bf16((batch, n_kv, total, 128), gen, device=DEV)
    v = random_bf16((batch, n_kv, total, 128), gen, device=DEV)
    # the query heads of a group share one query, so one key dominates all of them
    q_kv = random_bf16((batch, n_kv, 128), gen, device=DEV)
    q = q_kv[:, :, None, :].expand(batch, n_kv, group, 128).reshape(batch, n_q, 128).contiguous()
    sign = torch.where(q_kv.float() >= 0, 1.0, -1.0)
    beta = torch.from_numpy(mask.astype(np.float32)).to(DEV)
    live = [h for h in range(n_kv) if counts[h] > 0]
    specials = special_rows(n_sink, window, ctx, step)
    edges = middle_edges(n_sink, window, total, tiles=(total < 20000), before=edges_before)
    # each live pair takes a share of the edges (every edge in some pair)
    n_live_pairs = batch * len(live)
    expected = np.zeros((batch, n_q, 128), dtype=np.float64)
    vbits = 8 if bits == 0 else bits
    live_rank = 0
    for b in range(batch):
        for h in range(n_kv):
            if counts[h] > 0:
                share = edges[live_rank % n_live_pairs::n_live_pairs] if per_pair is None else \
                    list(rng.choice(edges, size=min(per_pair, len(edges)), replace=False))
                live_rank += 1
                rows = sorted(set(specials) | set(int(r) for r in share))
                key = NEEDLE_K * sign[b, h] * beta[h]        # kept channels only: one score everywhere
            else:
                mids = list(rng.choice(edges, size=min(16, len(edges)), replace=False))
                rows = sorted(set(specials) | set(int(r) for r in mids))
                key = NEEDLE_K * sign[b, h]                  # every channel (only full-width rows count)
            levels = np.stack([value_levels(rng, vbits) for _ in rows])
            values = to_values(levels, vbits)
            idx = torch.tensor(rows, device=DEV)
            k[b, h, idx] = key.to(torch.bfloat16)
            v[b, h, idx] = torch.from_numpy(values.astype(np.float32)).to(DEV).to(torch.bfloat16)
            full = np.array([r < n_sink or r >= total - window for r in rows])
            included = np.ones(len(rows), dtype=bool) if counts[h] > 0 else full
            assert included.any()
            expected[b, h * group:(h + 1) * group] = values[included].mean(axis=0)
    return mask, k, v, q, expected


def make_cache(mask, batch, n_q, n_sink, window, max_ctx, bits, paged, seed):
    kept_count, kept_idx = kept_from_mask(mask)
    extra = {}
    if paged:
        ppr = -(-max(0, max_ctx - n_sink - window) // 64)
        n_pages = batch * ppr + 3
        pick = np.random.default_rng(seed).permutation(n_pages)[:batch * ppr]
        extra = dict(n_pages=n_pages,
                     block_table=torch.from_numpy(pick.astype(np.int32).reshape(batch, ppr)).to(DEV))
    return dac.LayerCache(kept_count.tolist(), torch.from_numpy(kept_idx).to(DEV), batch, n_q,
                          mask.shape[0], n_sink, window, max_ctx, device=DEV, quant_bits=bits,
                          **extra)


def run_case(batch, n_q, counts, n_sink, window, ctx, step, bits, paged, seed, per_pair=None,
             oracle_pairs=2, edges_before=True):
    case("needles", batch, n_q, counts, n_sink, window, ctx, "step" if step else "decode",
         f"{bits}-bit" if bits else "bf16", "paged" if paged else "contiguous")
    mask, k, v, q, expected = build_needles(batch, n_q, counts, n_sink, window, ctx, step, bits,
                                            seed, per_pair, edges_before)
    cache = make_cache(mask, batch, n_q, n_sink, window, ctx + 2, bits, paged, seed)
    dac.leank_pack_k(cache, k[:, :, :ctx].contiguous(), v[:, :, :ctx].contiguous())
    if step:
        out = dac.leank_decode_step(cache, q, k[:, :, ctx].contiguous(), v[:, :, ctx].contiguous())
    else:
        out = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert_close(got, expected, "needle mean")
    # the construction itself, against the oracle on a few (batch row, head)
    group = n_q // len(counts)
    pairs = [(0, 0), (batch - 1, n_q - 1)] + [(batch // 2, h * group) for h in range(len(counts))
                                              if counts[h] == 0][:1]
    pairs = pairs[:oracle_pairs + 1]
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    ref = (oracle.decode_q(qb, kb, vb, mask, n_sink, window, bits, pairs=pairs) if bits
           else oracle.decode(qb, kb, vb, mask, n_sink, window, pairs=pairs))
    assert_close(np.array([expected[b, j] for b, j in pairs]), ref, "needle mean vs oracle")
    assert_close(np.array([got[b, j] for b, j in pairs]), ref, "needle output vs oracle")


@pytest.mark.parametrize("step", [False, True], ids=["decode", "step"])
@pytest.mark.parametrize("bits,paged", [(0, False), (0, True), (4, False), (8, False), (4, True)],
                         ids=["bf16", "bf16-paged", "4bit", "8bit", "4bit-paged"])
def test_needles_llama_b64_4k(bits, paged, step):
    run_case(64, 32, LLAMA_COUNTS, 64, 512, 4096, step, bits, paged, seed=11 + bits + paged,
             per_pair=48)


@pytest.mark.parametrize("step", [False, True], ids=["decode", "step"])
@pytest.mark.parametrize("bits,paged", [(0, False), (0, True), (4, False), (8, False)],
                         ids=["bf16", "bf16-paged", "4bit", "8bit"])
def test_needles_128k_b4(bits, paged, step):
    run_case(4, 32, LONG_COUNTS, 64, 2048, 131072, step, bits, paged, seed=21 + bits + paged,
             oracle_pairs=1)


@pytest.mark.parametrize("bits", [0, 4])
def test_needles_128k_b1_one_live_head(bits):
    """One live pair split into hundreds of items, merged over several
    channel slices of the workgroup combine: a needle at every 64-row edge
    of its middle, so every item holds some, and a lost or doubled record
    shows."""
    run_case(1, 32, [0, 0, 64, 0, 0, 0, 0, 0], 64, 2048, 131072, True, bits, False,
             seed=41 + bits, oracle_pairs=1, edges_before=False)


def test_needles_step_at_group_edge_q4():
    """A 4-bit step whose appended middle row completes a K group (the call
    that runs the append kernel first), at the Llama shape."""
    # the leaving token becomes middle row ctx - window - n_sink; 63 mod 64 completes the group
    ctx = 64 + 512 + 64 * 55 + 63
    run_case(64, 32, LLAMA_COUNTS, 64, 512, ctx, True, 4, False, seed=31, per_pair=48)


def test_needles_512_batch_rows():
    """Thousands of (batch row, KV head) pairs in one call: the combine's grid
    and the record offsets of the last batch rows."""
    run_case(512, 16, [32, 0, 64, 32, 0, 96, 32, 128], 4, 32, 300, True, 0, False, seed=71,
             per_pair=8)
