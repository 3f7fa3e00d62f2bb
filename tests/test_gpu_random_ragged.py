"""Seeded random ragged batches against the CPU oracle, across every cache kind.

Each case draws a layer shape and a cache kind as tests/test_gpu_random.py
does, then gives every batch row its own length (empty rows, rows inside the
sink and window, rows deep into the middle), prefills the rows with
`leank_pack_k_rows`, and checks either `leank_decode_attn_rows` over those
lengths or a fused `leank_decode_step_rows` that appends one token per row at
its own position, against the oracle's attention over each row's own tokens
(`oracle.decode`, or `oracle.decode_q` over the low-bit streams) on sampled
query heads.  A row of length 0 must give zeros.
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
N_CASES = 20


def draw(i):
    rng = np.random.default_rng(20261205 + i)
    group = int(rng.integers(1, 9))
    n_kv = int(rng.choice([1, 2, 4, 8, 12]))
    counts = [int(c) for c in rng.choice([0, 8, 16, 32, 64, 128], size=n_kv)]
    if not any(counts):
        counts[int(rng.integers(n_kv))] = 32
    n_sink = int(rng.choice([0, 4, 64]))
    window = int(rng.choice([1, 16, 256]))
    batch = int(rng.integers(2, 7))
    l_max = int(rng.integers(n_sink + window + 200, n_sink + window + 5000))
    lengths = [int(x) for x in rng.integers(0, l_max + 1, size=batch)]
    # an empty row, a row inside the sink and window, and a row at the maximum
    lengths[0] = 0 if i % 2 == 0 else 1
    lengths[1 % batch] = min(l_max, int(rng.integers(1, n_sink + window + 2)))
    lengths[-1] = l_max
    return dict(group=group, counts=counts, n_sink=n_sink, window=window, lengths=lengths,
                kind=KINDS[i % len(KINDS)], step=bool(i % 2), seed=20261205 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_ragged_layer(i):
    c = draw(i)
    print("CASE random ragged", i, c, flush=True)
    rng = np.random.default_rng(c["seed"])
    mask = mask_with_counts(rng, c["counts"])
    n_kv = mask.shape[0]
    n_q = n_kv * c["group"]
    lengths = c["lengths"]
    batch, l_max = len(lengths), max(lengths)
    cache, bits = build_kind(c["kind"], mask, batch, n_q, c["n_sink"], c["window"], l_max + 2, c["seed"])
    gen = torch.Generator(device=DEV).manual_seed(c["seed"])
    k = random_bf16((batch, n_kv, l_max + 1, 128), gen, scale=1.5)
    v = random_bf16((batch, n_kv, l_max + 1, 128), gen)
    q = random_bf16((batch, n_q, 128), gen)
    pos0 = torch.zeros(batch, dtype=torch.int64, device=DEV)
    cnt = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    dac.leank_pack_k_rows(cache, k[:, :, :l_max].contiguous(), v[:, :, :l_max].contiguous(), pos0, cnt)
    if c["step"]:
        at = torch.tensor(lengths, dtype=torch.int64, device=DEV)
        k_new = torch.stack([k[b, :, lengths[b]] for b in range(batch)]).contiguous()
        v_new = torch.stack([v[b, :, lengths[b]] for b in range(batch)]).contiguous()
        out = dac.leank_decode_step_rows(cache, q, k_new, v_new, at, max_ctx_len=l_max + 1)
        tokens = [n + 1 for n in lengths]
    else:
        ctx = torch.tensor(lengths, dtype=torch.int32, device=DEV)
        out = dac.leank_decode_attn_rows(cache, q, ctx, max_ctx_len=l_max)
        tokens = list(lengths)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    for b, t in enumerate(tokens):
        if t == 0:
            assert np.all(got[b] == 0.0), f"row {b}: an empty row must give zeros"
            continue
        heads = sorted({int(rng.integers(n_q)) for _ in range(6)} | {0, n_q - 1})
        pairs = [(0, j) for j in heads]
        args = (qb[b:b + 1], kb[b:b + 1, :, :t], vb[b:b + 1, :, :t], mask, c["n_sink"], c["window"])
        ref = oracle.decode_q(*args, bits, pairs=pairs) if bits else oracle.decode(*args, pairs=pairs)
        assert_close(np.stack([got[b, j] for j in heads]), ref, f"random ragged case {i} row {b} ({t} tokens)")
