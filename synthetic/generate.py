"""Seeded generators: alpha (numpy, host) and q / K / V (torch, any device)."""

import numpy as np
import torch

KIND_Q, KIND_K, KIND_V, KIND_KSCALE, KIND_STEPS_K, KIND_STEPS_V, KIND_STEPS_Q = 1, 2, 3, 4, 5, 6, 7


def seed_for(cfg_index, layer, kind, step=0):
    """Deterministic 63-bit seed per (workload, layer, tensor kind, step)."""
    x = (cfg_index + 1) * 0x9E3779B1
    x = (x * 1_000_003 + layer + 1) & ((1 << 63) - 1)
    x = (x * 1_000_033 + kind) & ((1 << 63) - 1)
    x = (x * 1_000_037 + step + 1) & ((1 << 63) - 1)
    return x


def alpha_for(cfg, seed=None, shape=None):
    """alpha float32 [L, H_kv, d] following the workload's recipe."""
    n_layers, n_heads, d = shape or (cfg.n_layers, cfg.n_kv_heads, cfg.head_dim)
    rng = np.random.default_rng(cfg.alpha_seed if seed is None else seed)
    u = np.abs(rng.standard_normal((n_layers, n_heads, d)))
    f = 0.2 + 0.8 * (np.arange(d) % 64) / 63.0
    if cfg.alpha_mode == "uniform":
        g = rng.uniform(0.05, 1.0, size=(n_layers, n_heads))
    elif cfg.alpha_mode == "dead":
        g = rng.uniform(cfg.live_lo, 1.0, size=n_layers * n_heads)
        dead = rng.permutation(n_layers * n_heads)[: cfg.n_dead]
        g[dead] = 0.01
        g = g.reshape(n_layers, n_heads)
    else:
        raise ValueError(cfg.alpha_mode)
    alpha = u * g[:, :, None] * f[None, None, :]
    return alpha.astype(np.float32)


def _normal(shape, seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_q(cfg, layer, step=0, device="cpu", batch=None):
    """q bf16 [B, Hq, d]."""
    b = cfg.batch if batch is None else batch
    x = _normal((b, cfg.n_q_heads, cfg.head_dim),
                seed_for(cfg.index, layer, KIND_Q, step), device)
    return x.to(torch.bfloat16)


def _k_scales(cfg, layer, device):
    if cfg.k_scale_sigma <= 0:
        return None
    z = _normal((cfg.n_kv_heads, cfg.head_dim), seed_for(cfg.index, layer, KIND_KSCALE), device)
    return torch.exp(cfg.k_scale_sigma * z)


def make_kv(cfg, layer, n_tokens=None, device="cpu", batch=None):
    """Prefill K, V bf16 [B, H_kv, n_tokens, d] (default n_tokens = cfg.ctx)."""
    b = cfg.batch if batch is None else batch
    t = cfg.ctx if n_tokens is None else n_tokens
    shape = (b, cfg.n_kv_heads, t, cfg.head_dim)
    k = _normal(shape, seed_for(cfg.index, layer, KIND_K), device)
    scales = _k_scales(cfg, layer, device)
    if scales is not None:
        k.mul_(scales[None, :, None, :])
    k = k.to(torch.bfloat16)
    v = _normal(shape, seed_for(cfg.index, layer, KIND_V), device).to(torch.bfloat16)
    return k, v


def make_step_kv(cfg, layer, step, device="cpu", batch=None):
    """K, V bf16 [B, H_kv, 1, d] of the token appended at decode step `step`."""
    b = cfg.batch if batch is None else batch
    shape = (b, cfg.n_kv_heads, 1, cfg.head_dim)
    k = _normal(shape, seed_for(cfg.index, layer, KIND_K, step + 1), device)
    scales = _k_scales(cfg, layer, device)
    if scales is not None:
        k.mul_(scales[None, :, None, :])
    v = _normal(shape, seed_for(cfg.index, layer, KIND_V, step + 1), device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def make_steps_kv(cfg, layer, n_steps, device="cpu", batch=None):
    """K, V bf16 [n_steps, B, H_kv, 1, d] of the tokens appended by a generation loop."""
    b = cfg.batch if batch is None else batch
    shape = (n_steps, b, cfg.n_kv_heads, 1, cfg.head_dim)
    k = _normal(shape, seed_for(cfg.index, layer, KIND_STEPS_K), device)
    scales = _k_scales(cfg, layer, device)
    if scales is not None:
        k.mul_(scales[None, None, :, None, :])
    v = _normal(shape, seed_for(cfg.index, layer, KIND_STEPS_V), device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def make_steps_q(cfg, step, device="cpu", batch=None):
    """q bf16 [L, B, Hq, d] for every layer at one generation step."""
    b = cfg.batch if batch is None else batch
    x = _normal((cfg.n_layers, b, cfg.n_q_heads, cfg.head_dim),
                seed_for(cfg.index, 0, KIND_STEPS_Q, step), device)
    return x.to(torch.bfloat16)


def bf16_bits(t):
    """Host numpy uint16 view of a bf16 tensor's bits."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
