"""Builds libleank.so (HIP, gfx950) in place, next to this file.

Run ``python -m decode_attention_channel_amd.build`` or call ``build()``.
Every call recompiles.  Objects go to ``_build/`` (not tracked).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libleank.so")
SOURCES = ["plan.hip", "mask.hip", "pack.hip", "quant.hip", "decode.hip", "analysis.hip"] + [f"decode_g{g}.hip" for g in range(1, 9)]
ARCH = "gfx950"

# Packed fp32 VALU forms (v_pk_fma_f32 and friends) are switched off for the
# device code; the host pass of hipcc warns that it does not know the feature.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
# The decode kernels hold no NaN for finite inputs (scores are finite or
# -inf, and every -inf difference is guarded), so their max reductions skip
# NaN quieting and each DPP step of a row reduction is one instruction.
SOURCE_FLAGS = {f"decode_g{g}.hip": ["-fno-honor-nans"] for g in range(1, 9)}


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose=False, extra_flags=()):
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objects = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objects.append(obj)
        jobs.append([hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags,
                     "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, os.cpu_count() or 2))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for fut in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            fut.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objects, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
