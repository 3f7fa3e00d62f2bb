"""bench.py's argument contract, checked without a GPU: requests it cannot
serve end with exit status 2 and a message before anything touches a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_other_workload_needs_skip_extras():
    r = _run("--workload", "qwen_b16_32k")
    assert r.returncode == 2
    assert "--skip-extras" in r.stderr


def test_unknown_workload_is_refused():
    r = _run("--workload", "no_such_workload")
    assert r.returncode == 2


def test_wave_combine_label_matches_the_kernels():
    import re

    sys.path.insert(0, ROOT)
    import bench

    text = open(os.path.join(ROOT, "decode_attention_channel_amd", "csrc", "decode_base.h")).read()
    assert int(re.search(r"#define LEANK_WAVE_COMBINE_ITEMS (\d+)", text).group(1)) == \
        bench.WAVE_COMBINE_ITEMS


def test_oracle_sampler_on_host_arrays():
    """The CPU baseline's sampler: seeded random (batch row, KV head) units,
    widening timed apart, scaled to the whole layer."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench

    rng = np.random.default_rng(3)
    q = rng.integers(0, 1 << 15, size=(2, 4, 128)).astype(np.uint16) & 0x3FFF
    k = rng.integers(0, 1 << 15, size=(2, 2, 40, 128)).astype(np.uint16) & 0x3FFF
    mask = np.ones((2, 128), dtype=np.uint8)
    mask[1] = 0
    attend, widen, n, units = bench.oracle_units(q, k, k, mask, 4, 8, target_seconds=0.0)
    assert n == 1 and units == 4 and attend > 0 and widen > 0
    attend, widen, n, units = bench.oracle_units(q, k, k, mask, 4, 8, target_seconds=60.0)
    assert n == units == 4
    threads, n_cpu, n_aff = bench.cpu_threads()
    assert 1 <= threads <= n_aff <= n_cpu
