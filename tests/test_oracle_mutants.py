"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Every mutant is a one-spot textual change of the oracle's source -- a dropped
term, an off-by-one boundary, a wrong index or sign, an inverted mask -- run
on the CPU in a throw-away module.  The real oracle is never modified.
"""

import inspect
import types

import pytest

import oracle.leank_oracle as real
from tests import oracle_pins

MUTANTS = [
    ("a pair asked twice answered in its last row only",
     "index.setdefault(tuple(pair), []).append(n)",
     "index[tuple(pair)] = n"),
    ("softmax scale from kept channels",
     "s = (keys @ qv) * scale",
     "s = (keys @ qv) / np.sqrt(max(1.0, beta.sum()))"),
    ("GQA head mapping modulo",
     "by_kv.setdefault((b, j // group), [])",
     "by_kv.setdefault((b, j % n_heads), [])"),
    ("dead head scores its middle as zero",
     "if live and mid_rows.size:",
     "if mid_rows.size:"),
    ("local window one token short",
     "local_begin = max(n_sink, ctx_len - window)",
     "local_begin = max(n_sink, ctx_len - window + 1)"),
    ("sink one token long",
     "sink = range(0, min(n_sink, ctx_len))",
     "sink = range(0, min(n_sink + 1, ctx_len))"),
    ("inverted channel mask",
     "keys_mid = get_k(b, h, mid_rows) * beta",
     "keys_mid = get_k(b, h, mid_rows) * (1.0 - beta)"),
    ("mask applied to full-width rows too",
     "keys_full = get_k(b, h, full_rows)",
     "keys_full = get_k(b, h, full_rows) * np.asarray(mask[h], dtype=np.float64)"),
    ("threshold rank floored",
     "return -((-(n - 1) * prune_pct) // 100)",
     "return ((n - 1) * prune_pct) // 100"),
    ("threshold percentile of the keep ratio",
     "threshold = ordered[prune_rank(n, prune_pct)]",
     "threshold = ordered[prune_rank(n, 100 - prune_pct)]"),
    ("kept count rounded up to the alignment",
     "n_keep = (n_keep // align) * align",
     "n_keep = -(-n_keep // align) * align"),
    ("strict threshold comparison",
     "n_keep = int(np.count_nonzero(a >= threshold))",
     "n_keep = int(np.count_nonzero(a > threshold))"),
    ("top-k ties towards the higher channel",
     "key=lambda c: (-a[c], c)",
     "key=lambda c: (-a[c], -c)"),
    ("kept channels left in importance order",
     "kept = sorted(by_importance[:n_keep])",
     "kept = by_importance[:n_keep]"),
    ("ring slot shifted by one",
     "return n_sink + (pos - n_sink) % window",
     "return n_sink + (pos - n_sink + 1) % window"),
    ("dead head keeps middle V",
     "v_mid.append(v_bits[:, head][:, mid].copy() if c > 0 else None)",
     "v_mid.append(v_bits[:, head][:, mid].copy())"),
    ("middle rows shifted by one",
     "mid = np.asarray(list(middle), dtype=np.int64)",
     "mid = np.asarray(list(middle), dtype=np.int64) + 1"),
    ("cache size without the K/V factor",
     "return 2 * n_layers * n_heads * head_dim * n_tokens * batch * bytes_per_elem",
     "return n_layers * n_heads * head_dim * n_tokens * batch * bytes_per_elem"),
    ("middle V counted for dead heads",
     "live = sum(1 for c in kept if c > 0)",
     "live = len(kept)"),
    ("retention counts one channel of the pair",
     "per_pair = (rows[:, :half] + rows[:, half:]) / 2.0",
     "per_pair = rows[:, :half]"),
    ("w_hf from the low-frequency end",
     "hf = a[..., :n_hf_pairs].sum(axis=-1) + a[..., half:half + n_hf_pairs].sum(axis=-1)",
     "hf = a[..., half - n_hf_pairs:half].sum(axis=-1) + a[..., d - n_hf_pairs:].sum(axis=-1)"),
    ("ties ranked by position",
     "            ranks[order[k]] = (i + j) / 2.0 + 1.0",
     "            ranks[order[k]] = k + 1.0"),
    ("exp without the max shift, weights unnormalised",
     "put(b, j, (w @ vals) / w.sum())",
     "put(b, j, (w @ vals) / len(w))"),
    ("quantization rounds down",
     "raw = np.rint((x - lo) / scale)",
     "raw = np.floor((x - lo) / scale)"),
    ("2^bits quantization steps",
     "levels = np.float32(2 ** bits - 1)",
     "levels = np.float32(2 ** bits)"),
    ("K quantized per token",
     "quantize_asym(k32.reshape(n_full, group, c), bits, axis=1)",
     "quantize_asym(k32.reshape(n_full, group, c), bits, axis=2)"),
    ("V quantized per channel",
     "v_codes, v_scale, v_lo = quantize_asym(v32, bits, axis=1)",
     "v_codes, v_scale, v_lo = quantize_asym(v32, bits, axis=0)"),
    ("minimum not added back",
     "            + np.asarray(lo, dtype=np.float64))",
     "            + 0.0 * np.asarray(lo, dtype=np.float64))"),
    ("quantized attention reads exact middle V",
     "v = dequantize(kq[\"v_codes\"], kq[\"v_scale\"][:, None], kq[\"v_lo\"][:, None])",
     "v = bf16_bits_to_f64(v_bits[b, h][middle_pos])"),
    ("quantization rounds half-way values up",
     "raw = np.rint((x - lo) / scale)",
     "raw = np.floor((x - lo) / scale + 0.5)"),
    ("low-bit pack quantizes batch row 0 for every row",
     "mid_q.append([quantize_middle(kp[b], ref[\"v_mid\"][head][b], bits, group)",
     "mid_q.append([quantize_middle(kp[0], ref[\"v_mid\"][head][0], bits, group)"),
    ("low-bit pack pairs every head's K with the first live head's V",
     "mid_q.append([quantize_middle(kp[b], ref[\"v_mid\"][head][b], bits, group)",
     "mid_q.append([quantize_middle(kp[b], [m for m in ref[\"v_mid\"] if m is not None][0][b], bits, group)"),
    ("widened entry point reads the first head's values",
     "lambda b, h, rows: v[b, h, rows],",
     "lambda b, h, rows: v[b, 0, rows],"),
    ("open K group left out of the byte count",
     "k = n_groups * group * c * bits // 8 + n_groups * c * 8 + n_stage * c * 2",
     "k = n_groups * group * c * bits // 8 + n_groups * c * 8"),
]


def _mutant_module(old, new):
    source = inspect.getsource(real)
    assert source.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
    module = types.ModuleType("oracle_mutant")
    exec(compile(source.replace(old, new), "<oracle-mutant>", "exec"), module.__dict__)
    return module


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    module = _mutant_module(old, new)
    caught_by = None
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(module)
        except Exception:  # an assertion or a crash both count as caught
            caught_by = pin.__name__
            break
    assert caught_by is not None, f"no pin catches: {name}"


def test_unmutated_copy_passes():
    module = _mutant_module("import numpy as np", "import numpy as np")
    for pin in oracle_pins.ALL_PINS:
        pin(module)
