"""Calls on two streams at once.

The library keeps no state between calls (the allocation-free step's scratch
aside), so fused steps on two caches issued alternately on two streams, with
no ordering between the streams, must give what the same steps give one
after the other on one stream: outputs and caches bit for bit, on two cache
kinds side by side.
"""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
from tests.gpu_cases import build_kind, mask_with_counts, random_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _buffers(cache):
    out = [cache.k_sl, cache.v_sl, cache.k_prun, cache.v_mid] + list(cache.quant.values())
    return out + ([cache.pool] if cache.pool is not None else [])


def test_steps_on_two_streams_match_one_stream():
    print("CASE two streams", flush=True)
    n_sink, window, group, batch, ctx, steps = 16, 64, 4, 4, 2000, 24
    kinds = ["bf16", "q4"]
    masks = [mask_with_counts(np.random.default_rng(91 + i), [32, 0, 64, 128]) for i in range(2)]
    gen = torch.Generator(device=DEV).manual_seed(91)
    data = []
    for i in range(2):
        k = random_bf16((batch, 4, ctx + steps, 128), gen)
        v = random_bf16((batch, 4, ctx + steps, 128), gen)
        q = random_bf16((batch, 4 * group, 128), gen)
        data.append((k, v, q))

    def fresh(i):
        cache, _ = build_kind(kinds[i], masks[i], batch, 4 * group, n_sink, window, ctx + steps + 1, 91 + i)
        for t in _buffers(cache):
            t.zero_()
        k, v, _ = data[i]
        dac.leank_pack_k(cache, k[:, :, :ctx].contiguous(), v[:, :, :ctx].contiguous())
        cache.workspace()
        return cache

    def step(cache, i, s, out, stream=None):
        k, v, q = data[i]
        dac.leank_decode_step(cache, q, k[:, :, ctx + s].contiguous(), v[:, :, ctx + s].contiguous(),
                              out=out, stream=stream)

    # one stream, one cache after the other
    ref = [fresh(0), fresh(1)]
    ref_out = [[torch.empty((batch, 4 * group, 128), dtype=torch.float32, device=DEV) for _ in range(steps)]
               for _ in range(2)]
    for i in range(2):
        for s in range(steps):
            step(ref[i], i, s, ref_out[i][s])
    torch.cuda.synchronize()

    # two streams, steps alternating between the caches
    par = [fresh(0), fresh(1)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    par_out = [[torch.empty_like(ref_out[0][0]) for _ in range(steps)] for _ in range(2)]
    for s in range(steps):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                # the inputs' slices are made on this stream, so the step sees them ready
                step(par[i], i, s, par_out[i][s], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        for s in range(steps):
            assert torch.equal(par_out[i][s], ref_out[i][s]), f"cache {i} step {s}"
        for a, b in zip(_buffers(par[i]), _buffers(ref[i])):
            assert torch.equal(a, b), f"cache {i} buffers"
