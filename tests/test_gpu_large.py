"""Caches whose middle streams pass 4 GiB.

Batch 16 with 8 live KV heads and 200K middle rows puts V_mid at 6.5 GB (in
a bf16 cache, or the page pool of a paged one), and 270K middle rows put an
8-bit cache's V codes at 4.4 GB, so the byte offsets of the last batch rows
lie above 2^32 in the pack kernels, the decode kernels and the fused step.
The outputs of the pairs at the highest offsets are checked against the
oracle, one KV head at a time from host copies of that head's rows only.
"""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import bf16_bits
from tests.gpu_cases import assert_close, build_kind, mask_with_counts, random_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _largest_stream_bytes(cache):
    tensors = [cache.v_mid, cache.k_prun] + list(cache.quant.values())
    if cache.pool is not None:
        tensors.append(cache.pool)
    return max(t.numel() * t.element_size() for t in tensors)


@pytest.mark.parametrize("kind,mid_rows", [("bf16", 200_000), ("paged", 200_000), ("q8", 270_000)])
def test_decode_and_step_past_4gib(kind, mid_rows):
    batch, n_kv, group, n_sink, window = 16, 8, 4, 64, 512
    ctx = n_sink + window + mid_rows
    print("CASE large cache", kind, batch, n_kv, ctx, flush=True)
    mask = mask_with_counts(np.random.default_rng(81), [32] * n_kv)
    cache, bits = build_kind(kind, mask, batch, n_kv * group, n_sink, window, ctx + 2, 81)
    assert _largest_stream_bytes(cache) > (4 << 30)
    gen = torch.Generator(device=DEV).manual_seed(81)
    k = torch.empty((batch, n_kv, ctx, 128), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    for b in range(batch):  # row by row: no float32 copy of the whole cache
        k[b] = random_bf16((n_kv, ctx, 128), gen, scale=1.5)
        v[b] = random_bf16((n_kv, ctx, 128), gen)
    q = random_bf16((batch, n_kv * group, 128), gen)
    k_new = random_bf16((batch, n_kv, 128), gen, scale=1.5)
    v_new = random_bf16((batch, n_kv, 128), gen)
    dac.leank_pack_k(cache, k, v)
    out_d = dac.leank_decode_attn(cache, q)
    out_s = dac.leank_decode_step(cache, q, k_new, v_new)
    torch.cuda.synchronize()
    got_d, got_s = out_d.cpu().numpy(), out_s.cpu().numpy()
    qb = bf16_bits(q)
    for b, h in ((batch - 1, n_kv - 1), (batch - 1, 0), (batch // 2, n_kv // 2), (0, 0)):
        kh = bf16_bits(torch.cat([k[b, h], k_new[b, h][None]])[None, None])
        vh = bf16_bits(torch.cat([v[b, h], v_new[b, h][None]])[None, None])
        qh = qb[b:b + 1, h * group:(h + 1) * group]
        if bits:
            ref_d = oracle.decode_q(qh, kh[:, :, :ctx], vh[:, :, :ctx], mask[h:h + 1], n_sink, window, bits)
            ref_s = oracle.decode_q(qh, kh, vh, mask[h:h + 1], n_sink, window, bits)
        else:
            ref_d = oracle.decode(qh, kh[:, :, :ctx], vh[:, :, :ctx], mask[h:h + 1], n_sink, window)
            ref_s = oracle.decode(qh, kh, vh, mask[h:h + 1], n_sink, window)
        assert_close(got_d[b, h * group:(h + 1) * group], ref_d[0], f"decode, row {b} head {h}")
        assert_close(got_s[b, h * group:(h + 1) * group], ref_s[0], f"step, row {b} head {h}")
