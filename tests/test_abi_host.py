"""Host-side checks of the C ABI: loading, exported symbols, plan logic, byte
accounting and argument errors that return before any kernel launch.

No call here launches a kernel: every failing call is rejected by the
host-side validation, and the success paths exercised are pure host code.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import decode_attention_channel_amd as dac
import oracle
from decode_attention_channel_amd import _lib
from synthetic import CONFIGS, alpha_for

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "leank.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(leank_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.lib()
    names = declared_functions()
    assert "leank_build_mask" in names and "leank_pack_k" in names and "leank_decode_attn" in names
    for name in names:
        assert hasattr(lib, name), name
    assert lib.leank_abi_version() == 7
    assert lib.leank_layer_cache_size() == ctypes.sizeof(_lib.LayerCacheDesc)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert dac.status_string(code).startswith("LEANK_")
    assert "unknown" in dac.status_string(42)


def test_plan_groups_heads_by_kept_count():
    kept = [32, 0, 64, 32, 128, 0, 96, 32]
    batch, max_ctx, n_sink, window = 3, 1003, 4, 61
    d = dac.leank_plan_layer(kept, batch, 16, 8, 128, n_sink, window, max_ctx)
    mid_cap = max_ctx - n_sink - window          # 938 rows
    v_mid_rows = -(-mid_cap // 8) * 8            # V is stored in blocks of 8 rows: 944
    slots = n_sink + window                      # 65 rows
    assert d.mid_capacity == mid_cap and d.n_live == 6
    order = [d.group_order[n] for n in range(8)]
    assert order == [4, 6, 2, 0, 3, 7, 1, 5]
    k_off = v_off = 0
    for h in order:
        if kept[h] == 0:
            assert d.k_prun_off[h] == -1 and d.v_mid_off[h] == -1
            continue
        assert d.k_prun_off[h] == k_off and d.v_mid_off[h] == v_off
        k_off += batch * mid_cap * kept[h]
        v_off += batch * v_mid_rows * 128
    assert d.k_prun_bytes == 2 * k_off and d.v_mid_bytes == 2 * v_off
    assert d.k_sl_bytes == batch * 8 * slots * 128 * 2
    assert d.v_sl_bytes == batch * 8 * 72 * 128 * 2
    assert [d.kept_count[h] for h in range(8)] == kept


@pytest.mark.parametrize("args,status", [
    (dict(head_dim=64), _lib.EUNSUPPORTED),
    (dict(kept=[12, 32]), _lib.EUNSUPPORTED),
    (dict(kept=[136, 32]), _lib.EINVAL),
    (dict(n_q=18), _lib.EUNSUPPORTED),      # 9 query heads per KV head
    (dict(n_q=3), _lib.EINVAL),             # not a multiple of n_kv
    (dict(n_sink=0, window=0), _lib.EINVAL),
    (dict(batch=0), _lib.EINVAL),
    (dict(max_ctx=0), _lib.EINVAL),
    (dict(n_sink=-1), _lib.EINVAL),
])
def test_plan_rejects(args, status):
    kw = dict(kept=[32, 64], batch=2, n_q=4, head_dim=128, n_sink=4, window=8, max_ctx=100)
    kw.update(args)
    with pytest.raises(dac.LeankError) as err:
        dac.leank_plan_layer(kw["kept"], kw["batch"], kw["n_q"], 2, kw["head_dim"],
                             kw["n_sink"], kw["window"], kw["max_ctx"])
    assert err.value.status == status


def test_plan_rejects_too_many_heads():
    with pytest.raises(dac.LeankError):
        dac.leank_plan_layer([32] * 65, 1, 65, 65, 128, 4, 8, 100)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_decode_bytes_match_oracle_accounting(cfg):
    _, kept_count, _ = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
    for layer in range(min(cfg.n_layers, 3)):
        kept = kept_count[layer].tolist()
        desc = dac.leank_plan_layer(kept, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, 128,
                                    cfg.n_sink, cfg.window, cfg.max_ctx)
        for ctx in sorted({1, cfg.n_sink, cfg.n_sink + cfg.window, cfg.n_sink + cfg.window + 1,
                           cfg.ctx, cfg.max_ctx}):
            if ctx < 1:
                continue
            got = dac.leank_decode_bytes(desc, ctx)
            assert got == oracle.decode_traffic_bytes(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads,
                                                       128, ctx, cfg.n_sink, cfg.window, kept)


def test_workspace_grows_with_context():
    rng = np.random.default_rng(5)
    for _ in range(20):
        n_kv = int(rng.integers(1, 9))
        group = int(rng.integers(1, 9))
        kept = [int(x) for x in rng.integers(0, 17, size=n_kv) * 8]
        batch = int(rng.integers(1, 70))
        n_sink, window = int(rng.integers(0, 70)), int(rng.integers(1, 700))
        max_ctx = int(rng.integers(1, 20000))
        desc = dac.leank_plan_layer(kept, batch, n_kv * group, n_kv, 128, n_sink, window, max_ctx)
        prev = 0
        for ctx in sorted(set(rng.integers(1, max_ctx + 1, size=40).tolist()) | {max_ctx}):
            ws = dac.leank_workspace_bytes(desc, ctx)
            assert ws >= prev and ws % 256 == 0
            prev = ws


def _fake_buffers(desc):
    # 16-byte aligned, never dereferenced: each call below fails validation first
    desc.kept_idx = desc.k_sl = desc.v_sl = desc.k_prun = desc.v_mid = 0x1000
    return desc


def test_calls_rejected_before_launch():
    L = _lib.lib()
    desc = dac.leank_plan_layer([32, 0], 2, 4, 2, 128, 4, 8, 100)
    ref = ctypes.byref(desc)
    # buffers not set
    assert L.leank_decode_attn(ref, 0x1000, 10, 0.1, 0x1000, 0x1000, 1 << 20, None) == _lib.EINVAL
    assert L.leank_pack_k(ref, 0x1000, 0x1000, 0, 1, None) == _lib.EINVAL
    _fake_buffers(desc)
    ws = dac.leank_workspace_bytes(desc, 100)
    assert L.leank_decode_attn(ref, 0x1000, 0, 0.1, 0x1000, 0x1000, ws, None) == _lib.EINVAL
    assert L.leank_decode_attn(ref, 0x1000, 101, 0.1, 0x1000, 0x1000, ws, None) == _lib.ECAPACITY
    assert L.leank_decode_attn(ref, 0x1000, 100, 0.1, 0x1000, 0x1000, ws - 1, None) == _lib.EWORKSPACE
    assert L.leank_decode_attn(ref, 0x1000, 100, 0.1, 0x1000, None, ws, None) == _lib.EWORKSPACE
    assert L.leank_decode_attn(ref, 0x1001, 100, 0.1, 0x1000, 0x1000, ws, None) == _lib.EINVAL
    assert L.leank_decode_attn(ref, 0x1000, 100, float("nan"), 0x1000, 0x1000, ws, None) == _lib.EINVAL
    assert L.leank_decode_attn(ref, 0x1000, 100, -1.0, 0x1000, 0x1000, ws, None) == _lib.EINVAL
    assert L.leank_pack_k(ref, 0x1000, 0x1000, 99, 2, None) == _lib.ECAPACITY
    assert L.leank_pack_k(ref, 0x1000, 0x1000, -1, 1, None) == _lib.EINVAL
    assert L.leank_pack_k(ref, 0x1000, 0x1008, 0, 1, None) == _lib.EINVAL
    assert L.leank_pack_k(ref, 0x1000, 0x1000, 5, 0, None) == _lib.OK   # empty append: no launch
    assert L.leank_decode_attn(None, 0x1000, 1, 0.1, 0x1000, 0x1000, ws, None) == _lib.EINVAL


def test_step_calls_rejected_before_launch():
    L = _lib.lib()
    desc = _fake_buffers(dac.leank_plan_layer([32, 0], 2, 4, 2, 128, 4, 8, 100))
    ref = ctypes.byref(desc)
    ws = dac.leank_workspace_bytes(desc, 100)
    p = 0x1000

    def step(pos, k=p, v=p, q=p, scale=0.1, out=p, work=p, nbytes=ws):
        return L.leank_decode_step(ref, q, k, v, pos, scale, out, work, nbytes, None)

    def step_rows(row_pos, max_len, k=p, nbytes=ws):
        return L.leank_decode_step_rows(ref, p, k, p, row_pos, max_len, 0.1, p, p, nbytes, None)

    assert step(100) == _lib.ECAPACITY         # the appended token would be row 101
    assert step(-1) == _lib.EINVAL
    assert step(5, k=None) == _lib.EINVAL
    assert step(5, v=0x1008) == _lib.EINVAL    # not 16-byte aligned
    assert step(5, q=0x1002) == _lib.EINVAL
    assert step(5, scale=0.0) == _lib.EINVAL
    assert step(5, work=None) == _lib.EWORKSPACE
    assert step(5, nbytes=16) == _lib.EWORKSPACE
    assert step_rows(None, 10) == _lib.EINVAL
    assert step_rows(p, 0) == _lib.EINVAL
    assert step_rows(p, 101) == _lib.ECAPACITY
    assert step_rows(p, 10, k=0x1004) == _lib.EINVAL
    assert L.leank_decode_step(None, p, p, p, 5, 0.1, p, p, ws, None) == _lib.EINVAL


def test_noalloc_step_rejected_before_launch():
    """The allocation-free step checks every argument before it looks up its
    device scratch (so these fail the same way with or without a GPU)."""
    L = _lib.lib()
    desc = _fake_buffers(dac.leank_plan_layer([32, 0], 2, 4, 2, 128, 4, 8, 100))
    ref = ctypes.byref(desc)
    p = 0x1000

    def step(pos, k=p, v=p, q=p, scale=0.1, out=p):
        return L.leank_decode_step_noalloc(ref, q, k, v, pos, scale, out, None)

    assert step(100) == _lib.ECAPACITY
    assert step(-1) == _lib.EINVAL
    assert step(5, k=None) == _lib.EINVAL
    assert step(5, v=0x1008) == _lib.EINVAL
    assert step(5, q=0x1002) == _lib.EINVAL
    assert step(5, out=None) == _lib.EINVAL
    assert step(5, scale=float("inf")) == _lib.EINVAL
    assert L.leank_decode_step_noalloc(None, p, p, p, 5, 0.1, p, None) == _lib.EINVAL
    unset = dac.leank_plan_layer([32, 0], 2, 4, 2, 128, 4, 8, 100)
    assert L.leank_decode_step_noalloc(ctypes.byref(unset), p, p, p, 5, 0.1, p, None) == _lib.EINVAL


def test_workspace_covers_a_step_at_the_same_context():
    """A step whose context after the append is n plans n - 1 regular rows
    plus one record per pair; the size for n must hold that."""
    rng = np.random.default_rng(9)
    for _ in range(20):
        n_kv = int(rng.integers(1, 9))
        kept = [int(x) for x in rng.integers(0, 17, size=n_kv) * 8]
        batch = int(rng.integers(1, 70))
        max_ctx = int(rng.integers(2, 20000))
        desc = dac.leank_plan_layer(kept, batch, n_kv, n_kv, 128, 4, 32, max_ctx)
        stride = 128 + 4   # floats per record at one query head per KV head
        for ctx in sorted(set(rng.integers(1, max_ctx + 1, size=10).tolist())):
            assert dac.leank_workspace_bytes(desc, ctx) >= batch * n_kv * stride * 4


def test_host_mask_feeds_the_plan_for_every_align():
    """leank_build_mask_host from host memory, for every align that divides
    128: an align the plan's kept-count quantum does not divide is refused
    (LEANK_EUNSUPPORTED); every other mask equals the oracle's bit for bit
    and each of its layers plans."""
    import torch

    for cfg in CONFIGS:
        alpha = alpha_for(cfg)
        for align in (1, 2, 4, 8, 16, 32, 64, 128):
            if align % _lib.CHANNEL_QUANTUM:
                with pytest.raises(dac.LeankError) as err:
                    dac.leank_build_mask(torch.from_numpy(alpha), cfg.prune_pct, align)
                assert err.value.status == _lib.EUNSUPPORTED
                continue
            mask, kept_count, kept_idx = dac.leank_build_mask(torch.from_numpy(alpha),
                                                              cfg.prune_pct, align)
            om, okc, oki = oracle.build_mask(alpha, cfg.prune_pct, align)
            assert np.array_equal(mask.numpy(), om), (cfg.name, align)
            assert np.array_equal(kept_count.numpy(), okc), (cfg.name, align)
            assert np.array_equal(kept_idx.numpy(), oki), (cfg.name, align)
            for layer in range(cfg.n_layers):
                dac.leank_plan_layer(kept_count[layer].tolist(), cfg.batch, cfg.n_q_heads,
                                     cfg.n_kv_heads, cfg.head_dim, cfg.n_sink, cfg.window,
                                     cfg.ctx + 1)


def test_host_mask_matches_oracle_on_ties_and_signs():
    import torch

    rng = np.random.default_rng(102)
    cases = [rng.integers(0, 5, size=(3, 5, 16)).astype(np.float32),
             np.full((2, 2, 32), 0.5, dtype=np.float32),
             rng.integers(0, 50, size=(2, 3, 1024)).astype(np.float32)]
    signed = rng.standard_normal((4, 4, 64)).astype(np.float32)
    signed[0, 0, :5] = [np.inf, -np.inf, 0.0, -0.0, 1e-45]
    signed[1, 2, :3] = [-0.0, 0.0, -0.0]
    cases.append(signed)
    for alpha in cases:
        for p in (0, 1, 33, 50, 70, 99, 100):
            for align in (8, 16, 32):
                if alpha.shape[2] % align:
                    continue
                mask, kc, ki = dac.leank_build_mask(torch.from_numpy(alpha), p, align)
                om, okc, oki = oracle.build_mask(alpha, p, align)
                assert np.array_equal(mask.numpy(), om) and np.array_equal(kc.numpy(), okc)
                assert np.array_equal(ki.numpy(), oki), (alpha.shape, p, align)
    nan = np.ones((1, 2, 128), dtype=np.float32)
    nan[0, 1, 3] = np.nan
    with pytest.raises(dac.LeankError) as err:
        dac.leank_build_mask(torch.from_numpy(nan), 50, 32)
    assert err.value.status == _lib.EINVAL


def test_build_mask_rejected_before_launch():
    L = _lib.lib()
    p = ctypes.c_void_p(0x1000)
    assert L.leank_build_mask(None, 1, 2, 128, 50, 32, p, p, p, None) == _lib.EINVAL
    assert L.leank_build_mask(p, 1, 2, 128, 101, 32, p, p, p, None) == _lib.EINVAL
    assert L.leank_build_mask(p, 1, 2, 128, -1, 32, p, p, p, None) == _lib.EINVAL
    assert L.leank_build_mask(p, 1, 2, 128, 50, 48, p, p, p, None) == _lib.EINVAL
    assert L.leank_build_mask(p, 1, 2, 128, 50, 0, p, p, p, None) == _lib.EINVAL
    assert L.leank_build_mask(p, 0, 2, 128, 50, 32, p, p, p, None) == _lib.EINVAL
    for align in (1, 2, 4):   # divides head_dim, but not a multiple of the kept-count quantum
        assert L.leank_build_mask(p, 1, 2, 128, 50, align, p, p, p, None) == _lib.EUNSUPPORTED
        assert L.leank_build_mask_host(p, 1, 2, 128, 50, align, p, p, p) == _lib.EUNSUPPORTED


def test_plan_layer_q_layout():
    kept = [32, 0, 64, 8]
    batch, max_ctx, n_sink, window = 3, 1000, 4, 61
    for bits in (4, 8):
        d = dac.leank_plan_layer_q(kept, batch, 8, 4, 128, n_sink, window, max_ctx, bits)
        mid_cap = max_ctx - n_sink - window
        g_rows = -(-mid_cap // 64) * 64
        v_rows = -(-mid_cap // 8) * 8
        assert d.quant_bits == bits and d.quant_group == 64
        assert d.k_prun_bytes == 0 and d.v_mid_bytes == 0
        off = dict(kq=0, kqp=0, ks=0, vq=0, vqp=0)
        for h in [d.group_order[n] for n in range(4)]:
            c = kept[h]
            if c == 0:
                assert d.k_q_off[h] == d.v_q_off[h] == d.k_stage_off[h] == -1
                continue
            assert (d.k_q_off[h], d.k_qp_off[h], d.k_stage_off[h], d.v_q_off[h], d.v_qp_off[h]) == \
                (off["kq"], off["kqp"], off["ks"], off["vq"], off["vqp"])
            off["kq"] += batch * g_rows * c * bits // 8
            off["kqp"] += batch * (g_rows // 64) * c * 2
            off["ks"] += batch * 64 * c
            off["vq"] += batch * v_rows * 128 * bits // 8
            off["vqp"] += batch * mid_cap * 2
        assert d.k_q_bytes == off["kq"] and d.k_qp_bytes == 4 * off["kqp"]
        assert d.k_stage_bytes == 2 * off["ks"] and d.v_q_bytes == off["vq"]
        assert d.v_qp_bytes == 4 * off["vqp"]


def test_plan_layer_q_rejects_other_widths():
    for bits in (1, 2, 3, 16):
        with pytest.raises(dac.LeankError) as err:
            dac.leank_plan_layer_q([32], 1, 1, 1, 128, 4, 8, 100, bits)
        assert err.value.status == _lib.EUNSUPPORTED


@pytest.mark.parametrize("bits", [4, 8])
def test_decode_bytes_q_match_oracle(bits):
    kept = [32, 0, 64, 128]
    n_sink, window, max_ctx = 4, 16, 700
    d = dac.leank_plan_layer_q(kept, 2, 8, 4, 128, n_sink, window, max_ctx, bits)
    for ctx in (1, 4, 20, 21, 83, 84, 85, 148, 700):
        assert dac.leank_decode_bytes(d, ctx) == oracle.decode_traffic_bytes_q(
            2, 8, 4, 128, ctx, n_sink, window, kept, bits), ctx


def test_plan_layer_paged_layout():
    kept = [32, 0, 64, 8]
    batch, max_ctx, n_sink, window, n_pages = 3, 1000, 4, 61, 50
    d = dac.leank_plan_layer_paged(kept, batch, 8, 4, 128, n_sink, window, max_ctx, n_pages)
    mid_cap = max_ctx - n_sink - window
    assert d.page_rows == 64 and d.pages_per_row == -(-mid_cap // 64) and d.n_pages == n_pages
    assert d.k_prun_bytes == 0 and d.v_mid_bytes == 0
    live = [h for h in (d.group_order[n] for n in range(4)) if kept[h] > 0]
    k_pre = 0
    for rank, h in enumerate(live):       # K of the live heads, then their V blocks
        assert d.k_prun_off[h] == 64 * k_pre
        assert d.v_mid_off[h] == 64 * (sum(kept) + rank * 128)
        k_pre += kept[h]
    assert d.k_prun_off[1] == -1 and d.v_mid_off[1] == -1
    assert d.page_bytes == 64 * (2 * sum(kept) + 256 * len(live))
    assert d.pool_bytes == n_pages * d.page_bytes


@pytest.mark.parametrize("bits", [4, 8])
def test_plan_layer_paged_q_layout(bits):
    """A paged low-bit page: K codes of the live heads in group order, their
    K (scale, min) pairs, their V code blocks, then their V row parameters;
    one 64-row K group per page; staging outside the pool."""
    kept = [32, 0, 64, 8]
    batch, max_ctx, n_sink, window, n_pages = 3, 1000, 4, 61, 50
    d = dac.leank_plan_layer_paged_q(kept, batch, 8, 4, 128, n_sink, window, max_ctx, n_pages, bits)
    mid_cap = max_ctx - n_sink - window
    assert d.quant_bits == bits and d.page_rows == 64 and d.pages_per_row == -(-mid_cap // 64)
    assert d.k_q_bytes == d.k_qp_bytes == d.v_q_bytes == d.v_qp_bytes == 0
    assert d.k_stage_bytes == batch * 64 * sum(kept) * 2
    live = [h for h in (d.group_order[n] for n in range(4)) if kept[h] > 0]
    kc = 64 * sum(kept) * bits // 8
    kp = 8 * sum(kept)
    vc = 64 * 128 * bits // 8
    k_pre = 0
    for rank, h in enumerate(live):
        assert d.k_q_off[h] == 64 * k_pre * bits // 8
        assert d.k_qp_off[h] * 4 == kc + 8 * k_pre
        assert d.v_q_off[h] == kc + kp + rank * vc
        assert d.v_qp_off[h] * 4 == kc + kp + len(live) * vc + rank * 512
        assert d.k_stage_off[h] == batch * 64 * k_pre
        k_pre += kept[h]
    assert d.page_bytes == kc + kp + len(live) * (vc + 512)
    assert d.pool_bytes == n_pages * d.page_bytes
    # every segment 16-byte aligned
    for h in live:
        assert d.k_q_off[h] % 16 == 0 and (d.k_qp_off[h] * 4) % 16 == 0
        assert d.v_q_off[h] % 16 == 0 and (d.v_qp_off[h] * 4) % 16 == 0
    # quant_bits 0 is the bf16 paged plan
    d0 = dac.leank_plan_layer_paged_q(kept, batch, 8, 4, 128, n_sink, window, max_ctx, n_pages, 0)
    d1 = dac.leank_plan_layer_paged(kept, batch, 8, 4, 128, n_sink, window, max_ctx, n_pages)
    assert bytes(d0) == bytes(d1)


def test_paged_q_layout_rejected_when_moved():
    L = _lib.lib()
    desc = dac.leank_plan_layer_paged_q([32, 0], 2, 4, 2, 128, 4, 8, 200, 4, 4)
    desc.kept_idx = desc.k_sl = desc.v_sl = desc.pool = desc.block_table = desc.k_stage = 0x1000
    ws = dac.leank_workspace_bytes(desc, 100)
    desc.v_q_off[0] += 16                  # not the canonical page layout (rejected before any launch)
    assert L.leank_decode_attn(ctypes.byref(desc), 0x1000, 100, 0.1, 0x1000, 0x1000, ws, None) == _lib.EINVAL


def test_paged_plan_and_calls_rejected():
    with pytest.raises(dac.LeankError):
        dac.leank_plan_layer_paged([32], 1, 1, 1, 128, 4, 8, 100, 0)   # no pages
    L = _lib.lib()
    desc = dac.leank_plan_layer_paged([32, 0], 2, 4, 2, 128, 4, 8, 100, 4)
    desc.kept_idx = desc.k_sl = desc.v_sl = 0x1000
    ws = dac.leank_workspace_bytes(desc, 100)
    # pool and block table missing
    assert L.leank_decode_attn(ctypes.byref(desc), 0x1000, 100, 0.1, 0x1000, 0x1000, ws, None) == _lib.EINVAL
    desc.pool = 0x1000
    assert L.leank_decode_attn(ctypes.byref(desc), 0x1000, 100, 0.1, 0x1000, 0x1000, ws, None) == _lib.EINVAL
    desc.block_table = 0x1000
    desc.k_prun_off[0] = 8                 # not the canonical page layout
    assert L.leank_decode_attn(ctypes.byref(desc), 0x1000, 100, 0.1, 0x1000, 0x1000, ws, None) == _lib.EINVAL
