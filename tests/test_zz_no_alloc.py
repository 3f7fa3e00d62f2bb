"""The allocation-free decode step, leank_decode_step_noalloc, against
leank_decode_step through the C ABI.

Two calls in a row, each on a pair of twin caches (same mask, same
prefill): the first on a Llama-3.1-8B-shaped cache (batch 16, context
4096), the second on a smaller one, so that the second call finds the
first call's records in the library's scratch.  Each must give the output
of leank_decode_step within 2e-3 + 1e-2 |ref| -- the kernels and the work
plan are the same, so the two agree bit for bit -- and leave the cache
holding exactly the oracle's packing of every token.  A call whose records
do not fit the scratch is rejected before any launch.
"""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from decode_attention_channel_amd import _lib
from synthetic import bf16_bits
from tests.gpu_cases import assert_cache_matches, assert_close, make_cache, mask_with_counts, random_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (batch, query heads, kept counts per KV head, sink, window, context, seed)
CALLS = [
    (16, 32, [32, 32, 32, 0, 32, 32, 32, 32], 64, 512, 4096, 1),
    (3, 8, [64, 0], 4, 16, 300, 2),
]


def case(*args):
    print("CASE", *args, flush=True)


def test_noalloc_step_matches_workspace_step():
    for batch, n_q, counts, n_sink, window, ctx, seed in CALLS:
        case("noalloc step", batch, n_q, counts, n_sink, window, ctx)
        mask = mask_with_counts(np.random.default_rng(seed), counts)
        n_kv = len(counts)
        gen = torch.Generator(device=DEV).manual_seed(500 + seed)
        k = random_bf16((batch, n_kv, ctx + 1, 128), gen)
        v = random_bf16((batch, n_kv, ctx + 1, 128), gen)
        q = random_bf16((batch, n_q, 128), gen)
        twins = [make_cache(mask, batch, n_q, n_sink, window, ctx + 4) for _ in range(2)]
        for c in twins:
            dac.leank_pack_k(c, k[:, :, :ctx].contiguous(), v[:, :, :ctx].contiguous())
        assert dac.leank_workspace_bytes(twins[0], ctx + 1) <= _lib.NOALLOC_SCRATCH_BYTES
        k_tok = k[:, :, ctx].contiguous()
        v_tok = v[:, :, ctx].contiguous()
        ref = dac.leank_decode_step(twins[0], q, k_tok, v_tok)
        got = torch.full_like(ref, float("nan"))
        dac.leank_decode_step_noalloc(twins[1], q, k_tok, v_tok, out=got)
        torch.cuda.synchronize()
        assert_close(got.cpu().numpy(), ref.cpu().numpy(), f"noalloc vs workspace step, ctx {ctx}")
        assert torch.equal(got, ref)
        kh, vh = bf16_bits(k), bf16_bits(v)
        for c in twins:
            assert c.length == ctx + 1
            assert_cache_matches(c, kh, vh, mask)
        # and the oracle, on a few query heads of the first and last batch rows
        pairs = [(0, 0), (0, n_q - 1), (batch - 1, n_q // 2)]
        want = oracle.decode(bf16_bits(q), kh, vh, mask, n_sink, window, pairs=pairs)
        assert_close(got.cpu().numpy()[[b for b, _ in pairs], [j for _, j in pairs]], want,
                     "noalloc step vs oracle")


def test_noalloc_step_rejects_calls_beyond_its_scratch():
    """Llama-3.1-8B-shaped batch 128 at context 4096 needs more records than
    the scratch holds: LEANK_EWORKSPACE, nothing written."""
    counts = [32, 32, 32, 0, 32, 32, 32, 32]
    mask = mask_with_counts(np.random.default_rng(3), counts)
    cache = make_cache(mask, 128, 32, 64, 512, 4100)
    case("noalloc step beyond scratch", dac.leank_workspace_bytes(cache, 4097))
    assert dac.leank_workspace_bytes(cache, 4097) > _lib.NOALLOC_SCRATCH_BYTES
    gen = torch.Generator(device=DEV).manual_seed(7)
    q = random_bf16((128, 32, 128), gen)
    tok = random_bf16((128, 8, 128), gen)
    out = torch.full((128, 32, 128), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(_lib.LeankError) as err:
        dac.leank_decode_step_noalloc(cache, q, tok, tok, pos=4096, out=out)
    assert err.value.status == _lib.EWORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
