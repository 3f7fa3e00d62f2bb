"""leank_decode_attn under HIP graph capture.

The decode call launches its two kernels on the caller's stream and makes no
allocation, copy or synchronisation, so a serving loop can capture it.  The
captured call is replayed several times, with eager calls and
synchronisations between the replays, and every replay must equal the eager
result bit for bit (the combine's summation order is fixed).
"""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
from tests.gpu_cases import assert_close, make_cache, mask_with_counts, oracle_outputs, random_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("ctx", [700, 20_000])
def test_decode_replayed_from_a_graph(ctx):
    print("CASE graph decode", ctx, flush=True)
    mask = mask_with_counts(np.random.default_rng(ctx), [32, 0, 64, 128])
    group = 4
    cache = make_cache(mask, 2, 4 * group, 16, 64, max_ctx=ctx + 1)
    gen = torch.Generator(device=DEV).manual_seed(ctx)
    k = random_bf16((2, 4, ctx, 128), gen)
    v = random_bf16((2, 4, ctx, 128), gen)
    q = random_bf16((2, 4 * group, 128), gen)
    dac.leank_pack_k(cache, k, v)
    eager = dac.leank_decode_attn(cache, q)
    torch.cuda.synchronize()
    assert_close(eager.cpu().numpy(), oracle_outputs(q, k, v, mask, 16, 64), "eager")

    ws = cache.workspace()
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dac.leank_decode_attn(cache, q, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dac.leank_decode_attn(cache, q, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        # eager work between replays, through the same workspace
        again = dac.leank_decode_attn(cache, q, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)
