"""The C ABI from plain C: include/leank.h compiles as C99 (pedantic) and a C
program linked against libleank.so gets the same host-side answers as the
Python binding.  Host-only entry points; no GPU."""

import ctypes
import os
import shutil
import subprocess

import pytest

import decode_attention_channel_amd as dac
from decode_attention_channel_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plain_c_consumer(tmp_path):
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    exe = tmp_path / "c_abi_host"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_host.c"),
           "-L", lib_dir, "-lleank", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    values, message = out.strip().split("\n")
    got = dict(kv.split("=") for kv in values.split())
    kept = [32, 0, 64, 8]
    d = dac.leank_plan_layer(kept, 3, 8, 4, 128, 4, 61, 1000)
    dq = dac.leank_plan_layer_q(kept, 3, 8, 4, 128, 4, 61, 1000, 4)
    dp = dac.leank_plan_layer_paged(kept, 3, 8, 4, 128, 4, 61, 1000, 50)
    dpq = dac.leank_plan_layer_paged_q(kept, 3, 8, 4, 128, 4, 61, 1000, 50, 8)
    assert int(got["abi"]) == _lib.lib().leank_abi_version()
    assert int(got["size"]) == ctypes.sizeof(_lib.LayerCacheDesc)
    assert int(got["status"]) == 0
    assert int(got["ws"]) == dac.leank_workspace_bytes(d, 1000)
    assert int(got["bytes"]) == dac.leank_decode_bytes(d, 1000)
    assert int(got["bytes_q"]) == dac.leank_decode_bytes(dq, 1000)
    assert int(got["page"]) == dp.page_bytes and int(got["page_q"]) == dpq.page_bytes
    assert int(got["bad"]) == _lib.EUNSUPPORTED
    assert message == dac.status_string(_lib.EUNSUPPORTED)
