"""Workload shapes for the synthetic inputs (see the package docstring)."""

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx: int                 # context length of the decode step (or of the prefill)
    n_sink: int
    window: int
    prune_pct: int
    align: int
    alpha_mode: str          # "uniform" or "dead"
    n_dead: int = 0          # heads over all layers given the small g
    live_lo: float = 0.05
    k_scale_sigma: float = 0.0
    decode_steps: int = 0    # generation-loop workloads: steps after the prefill
    alpha_seed: int = 0

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_ctx(self):
        return self.ctx + self.decode_steps


CONFIGS = [
    Config("tiny", 0, n_layers=1, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128,
           ctx=1024, n_sink=4, window=64, prune_pct=50, align=32,
           alpha_mode="uniform", alpha_seed=1000),
    Config("llama_b64_4k", 1, n_layers=1, batch=64, n_q_heads=32, n_kv_heads=8,
           head_dim=128, ctx=4096, n_sink=64, window=512, prune_pct=70, align=32,
           alpha_mode="dead", n_dead=1, live_lo=0.8, k_scale_sigma=0.5,
           alpha_seed=1100),
    Config("qwen_b16_32k", 2, n_layers=1, batch=16, n_q_heads=28, n_kv_heads=4,
           head_dim=128, ctx=32768, n_sink=64, window=1024, prune_pct=70, align=32,
           alpha_mode="dead", n_dead=1, live_lo=0.8, alpha_seed=1200),
    Config("llama32_b1_128k", 3, n_layers=32, batch=1, n_q_heads=32, n_kv_heads=8,
           head_dim=128, ctx=131072, n_sink=64, window=2048, prune_pct=80, align=64,
           alpha_mode="dead", n_dead=180, live_lo=0.9, alpha_seed=1300),
    Config("llama32_b64_gen", 4, n_layers=32, batch=64, n_q_heads=32, n_kv_heads=8,
           head_dim=128, ctx=4096, n_sink=64, window=512, prune_pct=70, align=32,
           alpha_mode="dead", n_dead=46, live_lo=0.8, decode_steps=1024,
           alpha_seed=1400),
]


def get_config(name_or_index):
    for cfg in CONFIGS:
        if cfg.name == name_or_index or cfg.index == name_or_index:
            return cfg
    raise KeyError(name_or_index)
