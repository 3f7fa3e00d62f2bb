"""Generation loop at full size: 32 layers of the Llama-3.1-8B attention
shape, batch 64, a 4096-token prefill and 1024 decode steps.  Every step
appends one token per layer (leank_pack_k, which moves the token leaving the
window into the pruned middle) and decodes (leank_decode_attn).

Checked against the CPU oracle: outputs of every layer at the first and the
last step and of layers 0, 15 and 31 every 128 steps, for sampled (batch
row, KV head) pairs; and the cache rows of those pairs bit for bit at the
same steps.
"""

import numpy as np
import pytest
import torch

import decode_attention_channel_amd as dac
import oracle
from synthetic import alpha_for, bf16_bits, get_config, make_kv, make_steps_kv, make_steps_q
from tests.gpu_cases import assert_cache_matches, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_generation_loop_full_size():
    cfg = get_config("llama32_b64_gen")
    n_steps = cfg.decode_steps
    print("CASE generation loop mask", flush=True)
    alpha = alpha_for(cfg)
    mask, kept_count, kept_idx = dac.leank_build_mask(torch.from_numpy(alpha).to(DEV),
                                                      cfg.prune_pct, cfg.align)
    om, okc, _ = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    assert np.array_equal(mask.cpu().numpy(), om)

    rng = np.random.default_rng(44)
    batches = sorted({0, cfg.batch - 1, int(rng.integers(1, cfg.batch - 1))})
    sample_pairs = [(b, h) for b in batches for h in range(cfg.n_kv_heads)]
    dense_layers = {0, 15, 31}
    check_steps = {0, n_steps - 1}
    periodic = {s for s in range(0, n_steps, 128)} | {n_steps - 1}

    caches, hist_k, hist_v, steps_k, steps_v = [], {}, {}, [], []
    for layer in range(cfg.n_layers):
        print("CASE generation loop prefill layer", layer, flush=True)
        cache = dac.LayerCache(kept_count[layer].cpu().tolist(), kept_idx[layer].contiguous(),
                               cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window,
                               cfg.max_ctx)
        k, v = make_kv(cfg, layer, device=DEV)
        dac.leank_pack_k(cache, k, v)
        sk, sv = make_steps_kv(cfg, layer, n_steps, device=DEV)
        steps_k.append(sk)
        steps_v.append(sv)
        kb, vb = bf16_bits(k), bf16_bits(v)
        skb, svb = bf16_bits(sk[:, :, :, 0]), bf16_bits(sv[:, :, :, 0])  # [S, B, H, d]
        for b, h in sample_pairs:
            hist_k[(layer, b, h)] = np.concatenate([kb[b, h], skb[:, b, h]], axis=0)
            hist_v[(layer, b, h)] = np.concatenate([vb[b, h], svb[:, b, h]], axis=0)
        caches.append(cache)
        del k, v
    torch.cuda.synchronize()

    got = {}
    out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=DEV)
    for step in range(n_steps):
        if step % 128 == 0:
            print("CASE generation loop step", step, flush=True)
        q_all = make_steps_q(cfg, step, device=DEV)
        for layer in range(cfg.n_layers):
            cache = caches[layer]
            dac.leank_pack_k(cache, steps_k[layer][step], steps_v[layer][step])
            dac.leank_decode_attn(cache, q_all[layer], out=out)
            want_out = step in check_steps or (layer in dense_layers and step in periodic)
            if want_out:
                qh = bf16_bits(q_all[layer])
                got[(step, layer)] = (out.cpu().numpy().copy(), qh)
            if layer in dense_layers and step in periodic:
                torch.cuda.synchronize()
                ctx = cfg.ctx + step + 1
                assert cache.length == ctx
                pairs = [p for p in sample_pairs]
                sel_k = np.stack([hist_k[(layer, b, h)][:ctx] for b, h in pairs])[:, None]
                sel_v = np.stack([hist_v[(layer, b, h)][:ctx] for b, h in pairs])[:, None]
                assert_cache_matches(cache, sel_k, sel_v, om[layer], pairs=pairs)
    torch.cuda.synchronize()

    print("CASE generation loop oracle", len(got), flush=True)
    for (step, layer), (out_np, qh) in sorted(got.items()):
        ctx = cfg.ctx + step + 1
        for b, h in sample_pairs:
            k1 = hist_k[(layer, b, h)][None, None, :ctx]
            v1 = hist_v[(layer, b, h)][None, None, :ctx]
            qg = qh[b:b + 1, h * cfg.group:(h + 1) * cfg.group]
            ref = oracle.decode(qg, k1, v1, om[layer][h:h + 1], cfg.n_sink, cfg.window)
            assert_close(out_np[b:b + 1, h * cfg.group:(h + 1) * cfg.group], ref,
                         f"step {step} layer {layer} pair {(b, h)}")
