"""Seeded synthetic inputs: determinism and the masks they realize."""

import numpy as np
import pytest
import torch

import oracle
from synthetic import CONFIGS, alpha_for, bf16_bits, get_config, make_kv, make_q, make_step_kv


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_alpha_recipe_and_realized_mask(cfg):
    alpha = alpha_for(cfg)
    assert alpha.dtype == np.float32
    assert alpha.shape == (cfg.n_layers, cfg.n_kv_heads, cfg.head_dim)
    assert np.array_equal(alpha, alpha_for(cfg))
    assert np.all(alpha >= 0)
    _, kept_count, _ = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    dead = int((kept_count == 0).sum())
    if cfg.alpha_mode == "dead":
        assert dead == cfg.n_dead
    # the realized prune ratio is at least the requested one (floor to the alignment)
    assert kept_count.sum() <= (100 - cfg.prune_pct) / 100 * alpha.size + kept_count.size


def test_tiny_mask_mixes_widths():
    cfg = get_config("tiny")
    _, kept_count, _ = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
    assert sorted(kept_count.ravel().tolist()) == [32, 64]


def test_qkv_generators_are_deterministic():
    cfg = get_config("tiny")
    k1, v1 = make_kv(cfg, 0, n_tokens=33)
    k2, v2 = make_kv(cfg, 0, n_tokens=33)
    assert k1.dtype == torch.bfloat16 and k1.shape == (1, 2, 33, 128)
    assert np.array_equal(bf16_bits(k1), bf16_bits(k2)) and np.array_equal(bf16_bits(v1), bf16_bits(v2))
    assert not np.array_equal(bf16_bits(k1), bf16_bits(v1))
    q = make_q(cfg, 0)
    assert q.shape == (1, 4, 128)
    ks, vs = make_step_kv(cfg, 0, 5)
    assert ks.shape == (1, 2, 1, 128)
    ks2, _ = make_step_kv(cfg, 0, 6)
    assert not np.array_equal(bf16_bits(ks), bf16_bits(ks2))


def test_k_channel_scales_only_where_configured():
    cfg = get_config("llama_b64_4k")
    k, _ = make_kv(cfg, 0, n_tokens=64, batch=2)
    per_channel = k.float().std(dim=(0, 2))      # [H, d]
    assert per_channel.max() / per_channel.min() > 2.0
