"""Seeded synthetic inputs for channel-pruned decode attention.

This module holds workload shapes and random-number recipes only -- none of
the method's arithmetic.  Both the CPU oracle's tests and the GPU path's
tests and benchmark draw their inputs from here, so the two sides always see
the same bits.

Workloads (one layer unless stated; head_dim 128 everywhere):

* ``tiny``            1 layer, B1, 4 q / 2 KV heads, T=1024 (S=4, W=64),
                      50% prune, align 32, g_h ~ U(0.05, 1).
* ``llama_b64_4k``    Llama-3.1-8B attention shape: 32 q / 8 KV heads,
                      B64, T=4096 (S=64, W=512), 70% prune, align 32,
                      K channel scales LogNormal(0, 0.5), 1 of 8 KV heads
                      fully pruned.
* ``qwen_b16_32k``    Qwen2.5-7B attention shape: 28 q / 4 KV heads, B16,
                      T=32768 (S=64, W=1024), 70% prune, align 32, 1 of 4
                      KV heads fully pruned.
* ``llama32_b1_128k`` 32 layers of the Llama shape, B1, T=131072 (S=64,
                      W=2048), 80% prune, align 64, 180 of 256 KV heads
                      fully pruned.
* ``llama32_b64_gen`` 32 layers of the Llama shape, B64, 4096-token
                      prefill then 1024 decode steps (S=64, W=512), 70%
                      prune, align 32, 46 of 256 KV heads fully pruned.

alpha recipe: alpha[l, h, c] = |N(0,1)| * g_h * f_c in float64, cast to
float32, with f_c = 0.2 + 0.8 * (c mod 64) / 63 rising over the rotate-half
channel-pair index.  ``uniform`` workloads draw g_h ~ U(0.05, 1); ``dead``
workloads give n_dead heads (a seeded choice) g = 0.01 and the others
g ~ U(live_lo, 1).

q / K / V recipe: float32 N(0, 1) from a torch generator on the target
device, seeded per (workload, layer, tensor kind, step), rounded to bf16.
Optional per-(KV head, channel) K scales exp(sigma * N(0, 1)) multiply K
before rounding.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .generate import (  # noqa: F401
    alpha_for,
    bf16_bits,
    make_q,
    make_kv,
    make_step_kv,
    make_steps_kv,
    make_steps_q,
    seed_for,
)
