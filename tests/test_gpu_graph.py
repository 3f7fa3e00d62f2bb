"""leank_decode_attn and the fused step under HIP graph capture.

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
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import (assert_close, build_kind, make_cache, mask_with_counts, oracle_outputs,
                             random_bf16)

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


def _buffers(cache):
    out = [cache.k_sl, cache.v_sl, cache.k_prun, cache.v_mid] + list(cache.quant.values())
    return out + ([cache.pool] if cache.pool is not None else [])


@pytest.mark.parametrize("kind", ["bf16", "q4", "paged"])
@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_step_captured_then_replayed_once(kind, noalloc):
    """A fused step (with a workspace, or leank_decode_step_noalloc) captured
    in a HIP graph and replayed once gives the eager step's output and cache,
    bit for bit, on a twin cache.  (A second replay would append at the same
    position again, so a step is replayed once.)"""
    ctx, n_sink, window, group = 700, 16, 64, 4
    print("CASE graph step", kind, "noalloc" if noalloc else "workspace", flush=True)
    mask = mask_with_counts(np.random.default_rng(77), [32, 0, 64, 128])
    batch, n_kv = 2, 4
    twins = []
    for _ in range(3):  # captured, eager, warm-up
        cache, _ = build_kind(kind, mask, batch, n_kv * group, n_sink, window, ctx + 4, 77)
        for t in _buffers(cache):
            t.zero_()
        twins.append(cache)
    gen = torch.Generator(device=DEV).manual_seed(77)
    k = random_bf16((batch, n_kv, ctx + 1, 128), gen)
    v = random_bf16((batch, n_kv, ctx + 1, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    for cache in twins:
        dac.leank_pack_k(cache, k[:, :, :ctx].contiguous(), v[:, :, :ctx].contiguous())
    k_new = k[:, :, ctx].contiguous()
    v_new = v[:, :, ctx].contiguous()
    outs = [torch.zeros((batch, n_kv * group, 128), dtype=torch.float32, device=DEV) for _ in twins]
    wss = [cache.workspace() for cache in twins]

    def step(i):
        if noalloc:
            dac.leank_decode_step_noalloc(twins[i], q, k_new, v_new, pos=ctx, out=outs[i])
        else:
            dac.leank_decode_step(twins[i], q, k_new, v_new, pos=ctx, out=outs[i], workspace=wss[i])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(2)  # warm-up on the third twin: the library and its scratch are set up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    step(1)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "replayed step output differs from the eager step"
    assert torch.equal(outs[1], outs[2])
    for a, b in zip(_buffers(twins[0]), _buffers(twins[1])):
        assert torch.equal(a, b), "replayed step left a different cache"
    if kind == "q4":
        ref = oracle.decode_q(bf16_bits(q), bf16_bits(k), bf16_bits(v), mask, n_sink, window, 4)
    else:
        ref = oracle_outputs(q, k, v, mask, n_sink, window)
    assert_close(outs[1].cpu().numpy(), ref, "eager step")
