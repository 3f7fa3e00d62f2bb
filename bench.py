"""Benchmark: one decode step of channel-pruned attention on one MI355X.

Workload (Llama-3.1-8B attention shape, one layer): 32 query / 8 KV heads,
head_dim 128, batch 64, context 4096 (64 sink tokens, 512-token window),
70% prune with align 32 on a seeded synthetic alpha, bf16 N(0,1) q/K/V with
LogNormal(0, 0.5) K channel scales.

A step is what a generation loop does per layer: append the new token's K/V
(the token leaving the window moves into the pruned middle) and run decode
attention over the whole cache, here as one leank_decode_step call (the
append runs inside the two decode kernels).  Each step appends one token,
so the context grows by one per step on each cache copy; copies rotate so
that consecutive steps read different HBM data (the copies together exceed
the 256 MB Infinity Cache many times over).

Reported on one JSON line: microseconds per step (value), the step's
roofline figures from HIP events on the launch stream, the same step as two
calls (leank_pack_k, then leank_decode_attn), the same step with the middle
held in 8-bit and 4-bit streams and in 64-row pages through a shuffled block
table, the same kernels at 0% pruning, the
Qwen2.5-7B-shaped cache, the 128K-token batch-1 workload (one layer, and all
32 layers per token), and the CPU oracle's time for the same step (a
baseline, not a target).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# the most items per (batch row, KV head) pair the one-wavefront combine merges
# (kWaveCombineItems in the decode kernels)
WAVE_COMBINE_ITEMS = 32
SHAPES = {
    "llama_b64_4k": "Llama-3.1-8B attention, one layer",
    "qwen_b16_32k": "Qwen2.5-7B attention, one layer",
    "llama32_b1_128k": "Llama-3.1-8B attention, layer 0 of the 32-layer 128K-token cache",
}
METRIC = ("pruned decode-attn µs/step & achieved HBM GB/s (% of 8 TB/s), "
          "Llama-3.1-8B shape")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=6, help="rotating cache copies")
    ap.add_argument("--workload", default="llama_b64_4k",
                    choices=["llama_b64_4k", "qwen_b16_32k", "llama32_b1_128k",
                             "llama32_b1_128k_model", "llama32_b64_gen"],
                    help="workload of the main line (llama_b64_4k is the headline).  With "
                         "--skip-extras another workload runs alone, for profiling: a one-layer "
                         "step (qwen_b16_32k, or llama32_b1_128k: its layer 0), every layer of "
                         "the 128K-token model per token (llama32_b1_128k_model, --steps "
                         "tokens), or the 32-layer generation loop (llama32_b64_gen, --gen-steps "
                         "steps)")
    ap.add_argument("--quant-bits", type=int, default=0, choices=[0, 4, 8],
                    help="one-layer workload alone: middle held in 4- or 8-bit streams")
    ap.add_argument("--paged", action="store_true",
                    help="one-layer workload alone: middle in 64-row pages (shuffled table)")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the main workload (no 0%% pruning, Qwen or CPU baseline)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle's sample of the headline step (the "
                         "other workloads' samples take fractions of it)")
    ap.add_argument("--gen-steps", type=int, default=1024,
                    help="decode steps of the 32-layer generation loop (the workload's 1024)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    return ap.parse_args()


def setup_caches(cfg, mask_counts, kept_idx_dev, k, v, copies, max_ctx, quant_bits=0,
                 paged=False):
    """`copies` caches holding the first ctx-1 tokens of k, v.  paged: the
    middle in 64-row pages, mapped through a seeded random block table."""
    import numpy as np
    import torch

    import decode_attention_channel_amd as dac

    caches = []
    for n in range(copies):
        extra = {}
        if paged:
            ppr = -(-max(0, max_ctx - cfg.n_sink - cfg.window) // 64)
            order = np.random.default_rng(77 + n).permutation(cfg.batch * ppr).astype(np.int32)
            extra = dict(n_pages=cfg.batch * ppr,
                         block_table=torch.from_numpy(order.reshape(cfg.batch, ppr)).to(k.device))
        cache = dac.LayerCache(mask_counts, kept_idx_dev, cfg.batch, cfg.n_q_heads,
                               cfg.n_kv_heads, cfg.n_sink, cfg.window, max_ctx,
                               quant_bits=quant_bits, **extra)
        dac.leank_pack_k(cache, k[:, :, : cfg.ctx - 1].contiguous(),
                         v[:, :, : cfg.ctx - 1].contiguous())
        cache.workspace()
        caches.append(cache)
    return caches


def gpu_lead(stream):
    """Queue about 0.2 ms of GPU spin on `stream` right before a timed region
    opens (after the synchronize that closes the warmup).  The region's start
    event then fires while the host is already submitting the region's first
    steps, so the host's submission of the first step (tens of microseconds
    through Python) is not counted as GPU time.  The spin is outside the
    region.  Measured on the Llama step: 20 timed steps gave 111.1-111.5 us
    per step without it against 109.7 us over 200."""
    import torch

    if not hasattr(torch.cuda, "_sleep"):  # a private torch helper; without it the region opens as before
        return
    with torch.cuda.stream(stream):
        torch.cuda._sleep(500_000)


def run_steps(cfg, caches, q, new_k, new_v, steps, warmup, fused=True):
    """Warm-up, then `steps` timed (append + decode) steps: one
    leank_decode_step call each (fused) or leank_pack_k + leank_decode_attn.
    Returns timings."""
    import torch

    import decode_attention_channel_amd as dac

    stream = torch.cuda.current_stream()
    n = len(caches)
    outs = [torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device) for _ in range(n)]

    def step(idx, events=None):
        cache = caches[idx % n]
        kk = new_k[idx % new_k.shape[0]]
        vv = new_v[idx % new_v.shape[0]]
        if events is not None:
            events[0].record(stream)
        if fused:
            dac.leank_decode_step(cache, q, kk, vv, out=outs[idx % n])
            if events is not None:
                events[1].record(stream)
                events[2].record(stream)
        else:
            dac.leank_pack_k(cache, kk, vv)
            if events is not None:
                events[1].record(stream)
            dac.leank_decode_attn(cache, q, out=outs[idx % n])
            if events is not None:
                events[2].record(stream)
        return cache.length

    for idx in range(warmup):
        step(idx)
    torch.cuda.synchronize()

    # throughput pass: exactly `steps` steps, events only around the pass
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    tp_ctx = []
    gpu_lead(stream)
    t_begin.record(stream)
    for s in range(steps):
        tp_ctx.append(step(warmup + s))
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_begin.elapsed_time(t_end)

    # instrumented pass: the same steps again with events around each launch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    ctxs = []
    base = warmup + steps
    for s in range(steps):
        ctxs.append(step(base + s, ev[s]))
    torch.cuda.synchronize()
    # fused: the whole step is one launch (ev 0 -> 2); unfused: append, then decode
    append_us = [ev[s][0].elapsed_time(ev[s][1]) * 1e3 for s in range(steps)] if not fused else []
    decode_us = [ev[s][0 if fused else 1].elapsed_time(ev[s][2]) * 1e3 for s in range(steps)]
    # algorithmic bytes of the attention over each throughput-pass step's context
    bytes_per = [dac.leank_decode_bytes(caches[(warmup + s) % n], tp_ctx[s]) for s in range(steps)]
    return {
        "total_ms": total_ms,
        "wall_s": wall,
        "append_us": append_us,
        "decode_us": decode_us,
        "ctx": ctxs,
        "throughput_ctx": tp_ctx,
        "decode_bytes": bytes_per,
    }


def summarize(t):
    """us_per_step: the throughput pass (HIP events around the whole timed
    region only); achieved_GBps: the attention's algorithmic bytes per step
    over that time.  events_*: the instrumented pass, with HIP events around
    each launch (they add several microseconds each, so they only show the
    split of an unfused step): the leank_decode_step call in a fused step,
    leank_pack_k and leank_decode_attn in an unfused one."""
    import numpy as np

    d = np.asarray(t["decode_us"])
    byt = float(np.mean(t["decode_bytes"]))
    us = t["total_ms"] * 1e3 / len(d)
    gbps = byt / (us * 1e-6) / 1e9
    return {
        "us_per_step": us,
        "decode_bytes_mean": byt,
        "achieved_GBps": gbps,
        "frac_of_peak": gbps / HBM_PEAK_GBPS,
        "events_launch_us_mean": float(d.mean()),
        "events_launch_us_p10": float(np.percentile(d, 10)),
        "events_launch_us_p50": float(np.percentile(d, 50)),
        "events_launch_us_p90": float(np.percentile(d, 90)),
        "events_append_us_mean": float(np.mean(t["append_us"])) if t["append_us"] else None,
        "ctx_range_throughput": [int(min(t["throughput_ctx"])), int(max(t["throughput_ctx"]))],
        "ctx_min": int(min(t["ctx"])),
        "ctx_max": int(max(t["ctx"])),
    }


def workload(cfg, prune_override=None, copies=6, steps=200, warmup=20, fused=True, quant_bits=0,
             paged=False):
    """Prepare one workload and time it.  prune_override=0 keeps every channel;
    quant_bits 4 or 8 holds the middle in low-bit streams; paged holds it in
    64-row pages through a block table."""
    import numpy as np
    import torch

    import decode_attention_channel_amd as dac
    from synthetic import alpha_for, make_kv, make_q, make_step_kv

    dev = torch.device("cuda:0")
    alpha = torch.from_numpy(alpha_for(cfg)).to(dev)
    prune = cfg.prune_pct if prune_override is None else prune_override
    mask, kept_count, kept_idx = dac.leank_build_mask(alpha, prune, cfg.align)
    counts = kept_count[0].cpu().tolist()
    k, v = make_kv(cfg, 0, device=dev)
    q = make_q(cfg, 0, device=dev)
    n_new = 8
    new = [make_step_kv(cfg, 0, s, device=dev) for s in range(n_new)]
    new_k = torch.stack([a for a, _ in new])
    new_v = torch.stack([b for _, b in new])
    max_ctx = cfg.ctx + (2 * steps + warmup) // copies + 2
    caches = setup_caches(cfg, counts, kept_idx[0].contiguous(), k, v, copies, max_ctx,
                          quant_bits, paged)
    torch.cuda.synchronize()
    timings = run_steps(cfg, caches, q, new_k, new_v, steps, warmup, fused=fused)
    res = summarize(timings)
    res["kept_count"] = counts
    res["dead_heads"] = int(sum(1 for c in counts if c == 0))
    res["realized_prune_pct"] = 100.0 * (1 - sum(counts) / (len(counts) * cfg.head_dim))
    res["cache_bytes_per_copy"] = int(caches[0].nbytes())
    del caches, k, v
    torch.cuda.empty_cache()
    return res


def whole_model(cfg, steps=20, warmup=3, prune_override=None):
    """All layers of a multi-layer workload per token: each layer has its own
    mask (one global threshold over every layer, as the mask is built),
    cache and query; a step is one leank_decode_step call per layer, in
    layer order.  Returns per-token time and the algorithmic bytes of every
    layer's attention."""
    import torch

    import decode_attention_channel_amd as dac
    from synthetic import alpha_for, make_kv, make_q, make_step_kv

    dev = torch.device("cuda:0")
    alpha = torch.from_numpy(alpha_for(cfg)).to(dev)
    prune = cfg.prune_pct if prune_override is None else prune_override
    mask, kept_count, kept_idx = dac.leank_build_mask(alpha, prune, cfg.align)
    counts_all = kept_count.cpu().tolist()
    max_ctx = cfg.ctx + steps + warmup + 2
    layers = []
    for layer in range(cfg.n_layers):
        cache = dac.LayerCache(counts_all[layer], kept_idx[layer].contiguous(), cfg.batch,
                               cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, max_ctx)
        k, v = make_kv(cfg, layer, n_tokens=cfg.ctx - 1, device=dev)
        dac.leank_pack_k(cache, k, v)
        del k, v
        cache.workspace()
        new = [make_step_kv(cfg, layer, s, device=dev) for s in range(steps + warmup)]
        out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
        layers.append((cache, make_q(cfg, layer, device=dev), new, out))
    torch.cuda.synchronize()

    def token(s):
        for cache, q, new, out in layers:
            dac.leank_decode_step(cache, q, new[s][0], new[s][1], out=out)

    for s in range(warmup):
        token(s)
    torch.cuda.synchronize()
    ctx0 = layers[0][0].length
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    gpu_lead(stream)
    t0.record(stream)
    for s in range(steps):
        token(warmup + s)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    # each step attends over its own context (the append comes first)
    byt = sum(dac.leank_decode_bytes(cache, ctx0 + s + 1)
              for cache, _, _, _ in layers for s in range(steps)) / steps
    live = sum(1 for row in counts_all for c in row if c > 0)
    res = {
        "us_per_token": us,
        "us_per_layer_mean": us / cfg.n_layers,
        "decode_bytes_per_token": byt,
        "achieved_GBps": byt / (us * 1e-6) / 1e9,
        "frac_of_peak": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "layers": cfg.n_layers,
        "live_kv_heads": live,
        "kv_heads": cfg.n_layers * cfg.n_kv_heads,
        "ctx_range_timed": [ctx0 + 1, ctx0 + steps],
        "steps": steps,
    }
    del layers
    torch.cuda.empty_cache()
    return res


def generation_loop(cfg, n_steps, prune_override=None, fused=True):
    """The 32-layer generation loop: every layer's cache prefilled with the
    workload's context, then n_steps decode steps in order, each appending
    one token per batch row to every layer and attending.  fused: one
    leank_decode_step per layer, in layer order.  Unfused: every layer's
    leank_pack_k, then every layer's leank_decode_attn, with HIP events
    around the two halves of each step (three events per step, so the split
    costs next to nothing).  Layers are independent of each other's output
    here, as the inputs are synthetic.  Returns per-step times and the
    attention's algorithmic bytes per step (every layer at its context)."""
    import numpy as np
    import torch

    import decode_attention_channel_amd as dac
    from synthetic import alpha_for, make_kv, make_q, make_step_kv

    dev = torch.device("cuda:0")
    alpha = torch.from_numpy(alpha_for(cfg)).to(dev)
    prune = cfg.prune_pct if prune_override is None else prune_override
    _, kept_count, kept_idx = dac.leank_build_mask(alpha, prune, cfg.align)
    counts_all = kept_count.cpu().tolist()
    max_ctx = cfg.ctx + n_steps + 2
    layers = []
    for layer in range(cfg.n_layers):
        cache = dac.LayerCache(counts_all[layer], kept_idx[layer].contiguous(), cfg.batch,
                               cfg.n_q_heads, cfg.n_kv_heads, cfg.n_sink, cfg.window, max_ctx)
        k, v = make_kv(cfg, layer, device=dev)
        dac.leank_pack_k(cache, k, v)
        del k, v
        cache.workspace()
        new = [make_step_kv(cfg, layer, s, device=dev) for s in range(4)]
        out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
        layers.append((cache, make_q(cfg, layer, device=dev), new, out))
    torch.cuda.synchronize()
    ctx0 = layers[0][0].length
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    split = []
    gpu_lead(stream)
    t0.record(stream)
    for s in range(n_steps):
        if fused:
            for cache, q, new, out in layers:
                dac.leank_decode_step(cache, q, new[s % 4][0], new[s % 4][1], out=out)
        else:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            for cache, q, new, out in layers:
                dac.leank_pack_k(cache, new[s % 4][0], new[s % 4][1])
            ev[1].record(stream)
            for cache, q, new, out in layers:
                dac.leank_decode_attn(cache, q, out=out)
            ev[2].record(stream)
            split.append(ev)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n_steps
    byt = float(np.mean([sum(dac.leank_decode_bytes(cache, ctx0 + s + 1) for cache, _, _, _ in layers)
                         for s in range(n_steps)]))
    res = {
        "ms_per_step": ms,
        "decode_bytes_per_step": byt,
        "achieved_GBps": byt / (ms * 1e-3) / 1e9,
        "frac_of_peak": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "floor_ms_at_peak": byt / (HBM_PEAK_GBPS * 1e9) * 1e3,
        "layers": cfg.n_layers,
        "batch": cfg.batch,
        "steps_timed": n_steps,
        "ctx_range_timed": [ctx0 + 1, ctx0 + n_steps],
        "live_kv_heads": sum(1 for row in counts_all for c in row if c > 0),
        "kv_heads": cfg.n_layers * cfg.n_kv_heads,
        "step": "leank_decode_step per layer (fused)" if fused else
                "leank_pack_k per layer, then leank_decode_attn per layer",
    }
    if split:
        res["pack_ms_per_step"] = float(np.mean([e[0].elapsed_time(e[1]) for e in split]))
        res["decode_ms_per_step"] = float(np.mean([e[1].elapsed_time(e[2]) for e in split]))
    del layers
    torch.cuda.empty_cache()
    return res


def cpu_threads():
    """Threads for the CPU oracle: the cores this process may run on (its
    affinity), capped by OMP_NUM_THREADS when set; BLAS is pinned to that.
    Returns (threads, os.cpu_count(), affinity size)."""
    n_cpu = os.cpu_count() or 1
    try:
        n_aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n_aff = n_cpu
    n = n_aff
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n, n_cpu, n_aff


def oracle_units(q_bits, k_bits, v_bits, mask, n_sink, window, target_seconds, seed=0):
    """The CPU oracle on one layer's decode, one (batch row, KV head) unit at
    a time in a seeded random order, until about target_seconds have passed
    (at least one unit).  Each unit's bf16 -> float64 widening and its
    attention (oracle.decode_f64) are timed apart.  Returns (seconds of
    attention per full layer, seconds of widening per full layer, units
    timed, units in the layer): the means over the units timed times the
    units in the layer (a uniform random sample, so unbiased)."""
    import numpy as np

    import oracle

    batch, n_q, _ = q_bits.shape
    n_kv = k_bits.shape[1]
    group = n_q // n_kv
    order = np.random.default_rng(seed).permutation(batch * n_kv)
    widen, attend = [], []
    t_all = time.perf_counter()
    for n in order:
        b, h = divmod(int(n), n_kv)
        t0 = time.perf_counter()
        qw = oracle.bf16_bits_to_f64(q_bits[b:b + 1, h * group:(h + 1) * group])
        kw = oracle.bf16_bits_to_f64(k_bits[b:b + 1, h:h + 1])
        vw = oracle.bf16_bits_to_f64(v_bits[b:b + 1, h:h + 1])
        t1 = time.perf_counter()
        oracle.decode_f64(qw, kw, vw, mask[h:h + 1], n_sink, window)
        t2 = time.perf_counter()
        widen.append(t1 - t0)
        attend.append(t2 - t1)
        if time.perf_counter() - t_all >= target_seconds:
            break
    units = batch * n_kv
    return float(np.mean(attend)) * units, float(np.mean(widen)) * units, len(attend), units


def _layer_bits(cfg, layer, n_tokens=None):
    """Host bf16 bits of one layer's synthetic q, K, V (generated on the GPU
    from the same seeds as the GPU workload) and its oracle mask row."""
    import torch

    from synthetic import bf16_bits, make_kv, make_q

    dev = torch.device("cuda:0")
    k, v = make_kv(cfg, layer, n_tokens=n_tokens, device=dev)
    q = make_q(cfg, layer, device=dev)
    out = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    del k, v
    torch.cuda.empty_cache()
    return out


def cpu_baselines(target_seconds):
    """The CPU oracle (plain float64 numpy, as it stands) on the host's cores,
    on bounded samples of the benchmark workloads.  The first entry is the
    headline's (the Llama-3.1-8B-shaped batch-64 4K step); the others are
    the Qwen2.5-7B-shaped batch-16 32K step, the 128K-token batch-1 model
    (per layer and per token) and the 32-layer generation loop (per step)."""
    import oracle
    from synthetic import alpha_for, get_config

    import contextlib

    threads, n_cpu, n_aff = cpu_threads()
    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(limits=threads)
    except ImportError:  # pragma: no cover
        limiter = contextlib.nullcontext()
    where = {"cores": threads, "host_cpus": n_cpu, "affinity_cpus": n_aff,
             "blas_threads": threads}
    res = {}
    with limiter:
        # headline: one layer step of the Llama workload
        cfg = get_config("llama_b64_4k")
        mask, _, _ = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
        qb, kb, vb = _layer_bits(cfg, 0)
        att, wid, n, units = oracle_units(qb, kb, vb, mask[0], cfg.n_sink, cfg.window,
                                          target_seconds)
        res["headline"] = dict(
            value=att * 1e6, unit="us/step", kind="oracle", **where,
            widening_us_per_step=wid * 1e6,
            sample=(f"{n} of the {units} (batch row, KV head) units of the {cfg.name} decode "
                    f"step (context {cfg.ctx}), in seeded random order, float64 attention "
                    f"(oracle.decode_f64) timed apart from the bf16 -> float64 widening; the "
                    f"mean per unit times {units}; {threads} BLAS threads"))
        del qb, kb, vb
        # Qwen2.5-7B-shaped step
        cfg = get_config("qwen_b16_32k")
        mask, _, _ = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
        qb, kb, vb = _layer_bits(cfg, 0)
        att, wid, n, units = oracle_units(qb, kb, vb, mask[0], cfg.n_sink, cfg.window,
                                          0.6 * target_seconds, seed=1)
        res["qwen_b16_32k"] = dict(value=att * 1e6, unit="us/step", widening_us_per_step=wid * 1e6,
                                   units_timed=n, units=units, **where)
        del qb, kb, vb
        # 128K-token batch-1 model: layers 0 and 1 timed, the token from
        # their per-head means (every live head of this model keeps the
        # same number of channels, so a head costs the same in every layer)
        cfg = get_config("llama32_b1_128k")
        mask, kept_count, _ = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
        live_t, dead_t, layers_us = [], [], []
        for layer in (0, 1):
            qb, kb, vb = _layer_bits(cfg, layer)
            for h in range(cfg.n_kv_heads):
                g = cfg.group
                t0 = time.perf_counter()
                qw = oracle.bf16_bits_to_f64(qb[:, h * g:(h + 1) * g])
                kw = oracle.bf16_bits_to_f64(kb[:, h:h + 1])
                vw = oracle.bf16_bits_to_f64(vb[:, h:h + 1])
                t1 = time.perf_counter()
                oracle.decode_f64(qw, kw, vw, mask[layer, h:h + 1], cfg.n_sink, cfg.window)
                t2 = time.perf_counter()
                (live_t if kept_count[layer, h] > 0 else dead_t).append(t2 - t1)
            del qb, kb, vb
        n_live = int((kept_count > 0).sum())
        n_dead = kept_count.size - n_live
        live_mean = sum(live_t) / len(live_t)
        dead_mean = sum(dead_t) / len(dead_t)
        layer0 = live_mean * int((kept_count[0] > 0).sum()) + dead_mean * int((kept_count[0] == 0).sum())
        res["llama32_b1_128k"] = dict(
            layer0_us=layer0 * 1e6, token_us=(live_mean * n_live + dead_mean * n_dead) * 1e6,
            unit="us", live_head_us=live_mean * 1e6, dead_head_us=dead_mean * 1e6, **where,
            sample=(f"every KV head of layers 0 and 1 at context {cfg.ctx} ({len(live_t)} live, "
                    f"{len(dead_t)} fully pruned), float64 attention only; the token as "
                    f"{n_live} live + {n_dead} fully pruned heads at those means"))
        # generation loop: layers 0 and 31 at the first and the last step
        cfg = get_config("llama32_b64_gen")
        mask, kept_count, _ = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
        per_layer = []
        for ctx in (cfg.ctx + 1, cfg.ctx + cfg.decode_steps):
            for layer in (0, cfg.n_layers - 1):
                qb, kb, vb = _layer_bits(cfg, layer, n_tokens=ctx)
                att, _, n, units = oracle_units(qb, kb, vb, mask[layer], cfg.n_sink, cfg.window,
                                                0.15 * target_seconds, seed=2 + layer)
                per_layer.append(att)
                del qb, kb, vb
        step = sum(per_layer) / len(per_layer) * cfg.n_layers
        res["llama32_b64_gen"] = dict(
            ms_per_step=step * 1e3, unit="ms/step", **where,
            sample=(f"layers 0 and {cfg.n_layers - 1} at contexts {cfg.ctx + 1} and "
                    f"{cfg.ctx + cfg.decode_steps}, sampled (batch row, KV head) units of each; the "
                    f"step as {cfg.n_layers} layers at their mean"))
    return res


def copy_calibration():
    """A plain device copy of known size (256 MiB read + 256 MiB written), run
    five times, so that memory counters of the same profile can be scaled."""
    import torch

    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read": n, "bytes_written": n, "launches": 5}


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_llama_b64_4k_counters.md")
KERNEL_SOURCES = ["decode_attention_channel_amd/csrc/decode_kernels.h",
                  "decode_attention_channel_amd/csrc/decode_base.h",
                  "decode_attention_channel_amd/csrc/tile_bf16.h",
                  "decode_attention_channel_amd/csrc/tile_lowbit.h",
                  "decode_attention_channel_amd/csrc/step_tokens.h",
                  "decode_attention_channel_amd/csrc/quant.h",
                  "decode_attention_channel_amd/csrc/decode_g4.hip",
                  "decode_attention_channel_amd/csrc/decode.hip",
                  "decode_attention_channel_amd/csrc/common.h",
                  "decode_attention_channel_amd/csrc/plan.hip"]


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode call from the committed counter summary, or None
    if the summary is missing or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_decode_call"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path; every figure is one GPU's.", file=sys.stderr)
        sys.exit(2)
    from synthetic import get_config

    alone = args.workload != "llama_b64_4k" or args.quant_bits or args.paged
    if alone and not args.skip_extras:
        print("--workload other than llama_b64_4k, --quant-bits and --paged profile one workload "
              "alone: add --skip-extras", file=sys.stderr)
        sys.exit(2)
    many_layers = args.workload in ("llama32_b1_128k_model", "llama32_b64_gen")
    cfg = get_config({"llama32_b1_128k_model": "llama32_b1_128k"}.get(args.workload, args.workload))
    headline = cfg.name == "llama_b64_4k" and not alone
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import decode_attention_channel_amd as dac

    dac.lib()  # fail loudly if the HIP library is missing
    torch.cuda.synchronize()
    if many_layers:
        if args.workload == "llama32_b64_gen":
            res = generation_loop(cfg, args.gen_steps)
        else:
            res = whole_model(cfg, steps=args.steps, warmup=args.warmup)
        if args.copy_calibration:
            res["copy_calibration"] = copy_calibration()
        print(json.dumps({"workload": args.workload, **res}), flush=True)
        return
    main_res = workload(cfg, copies=args.copies, steps=args.steps, warmup=args.warmup,
                        quant_bits=args.quant_bits, paged=args.paged)
    extras = {}
    if not args.skip_extras:
        unfused = workload(cfg, copies=args.copies, steps=args.steps, warmup=args.warmup,
                           fused=False)
        dense = workload(cfg, prune_override=0, copies=args.copies, steps=args.steps,
                         warmup=args.warmup)
        qwen_cfg = get_config("qwen_b16_32k")
        qwen = workload(qwen_cfg, copies=args.copies, steps=args.steps, warmup=args.warmup)
        qwen_dense = workload(qwen_cfg, prune_override=0, copies=max(2, args.copies // 2),
                              steps=args.steps, warmup=args.warmup)
        q8 = workload(cfg, copies=args.copies, steps=args.steps, warmup=args.warmup, quant_bits=8)
        q4 = workload(cfg, copies=args.copies, steps=args.steps, warmup=args.warmup, quant_bits=4)
        paged = workload(cfg, copies=args.copies, steps=args.steps, warmup=args.warmup, paged=True)
        paged_q4 = workload(cfg, copies=args.copies, steps=args.steps, warmup=args.warmup,
                            quant_bits=4, paged=True)
        long_cfg = get_config("llama32_b1_128k")
        long_ctx = workload(long_cfg, copies=args.copies, steps=args.steps, warmup=args.warmup)
        long_model = whole_model(long_cfg)
        long_model_dense = whole_model(long_cfg, prune_override=0)
        gen_cfg = get_config("llama32_b64_gen")
        gen = generation_loop(gen_cfg, args.gen_steps)
        gen_unfused = generation_loop(gen_cfg, args.gen_steps, fused=False)
        gen_dense = generation_loop(gen_cfg, args.gen_steps, prune_override=0)
        extras = {
            "unfused_pack_then_decode": unfused,
            "lowbit_middle_8bit": q8,
            "lowbit_middle_4bit": q4,
            "paged_middle_64row_pages": paged,
            "paged_lowbit_4bit": paged_q4,
            "dense_0pct": dense,
            "speedup_vs_0pct_step": dense["us_per_step"] / main_res["us_per_step"],
            "speedup_fused_vs_unfused_step": unfused["us_per_step"] / main_res["us_per_step"],
            "qwen_b16_32k": qwen,
            "qwen_b16_32k_dense_0pct": qwen_dense,
            "qwen_speedup_vs_0pct_step": qwen_dense["us_per_step"] / qwen["us_per_step"],
            "llama_b1_128k_layer0": long_ctx,
            "llama_b1_128k_all_32_layers": long_model,
            "llama_b1_128k_all_32_layers_dense_0pct": long_model_dense,
            "llama_b1_128k_speedup_vs_0pct_token": (long_model_dense["us_per_token"]
                                                     / long_model["us_per_token"]),
            "llama32_b64_generation_loop": gen,
            "llama32_b64_generation_loop_unfused": gen_unfused,
            "llama32_b64_generation_loop_dense_0pct": gen_dense,
            "generation_speedup_vs_0pct_step": gen_dense["ms_per_step"] / gen["ms_per_step"],
        }
    if args.copy_calibration:
        extras["copy_calibration"] = copy_calibration()
    cpu = None
    if not args.skip_extras:
        cpu_all = cpu_baselines(args.cpu_seconds)
        cpu = cpu_all.pop("headline")
        extras["cpu_oracle_other_workloads"] = cpu_all

    line = {
        "metric": METRIC,
        "value": main_res["us_per_step"],
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["us_per_step"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": cfg.name + (f"_{args.quant_bits}bit" if args.quant_bits else "")
                        + ("_paged" if args.paged else ""),
            "shape": SHAPES.get(cfg.name, cfg.name),
            "batch": cfg.batch,
            "n_q_heads": cfg.n_q_heads,
            "n_kv_heads": cfg.n_kv_heads,
            "head_dim": cfg.head_dim,
            "ctx": cfg.ctx,
            "ctx_range_timed": main_res["ctx_range_throughput"],
            "n_sink": cfg.n_sink,
            "window": cfg.window,
            "prune_pct": cfg.prune_pct,
            "align": cfg.align,
            "step": "leank_decode_step (append 1 token + decode attention, fused)",
            "cache_copies": args.copies,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": (f"leank_decode_step = decode_split_kernel<{cfg.group}> + its combine "
                       f"(decode_combine_wave_kernel<{cfg.group}> up to {WAVE_COMBINE_ITEMS} "
                       f"items per pair, else decode_combine_kernel<{cfg.group}>); "
                       "one launch pair per step, averaged over the timed steps"),
            "achieved": main_res["achieved_GBps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": main_res["frac_of_peak"],
            "traffic": measured_traffic() if headline else None,
            "bytes_per_launch": main_res["decode_bytes_mean"],
            "launch_us": main_res["us_per_step"],
        },
        "cpu_baseline": cpu,
        "pruned": main_res,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
