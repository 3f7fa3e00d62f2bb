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
