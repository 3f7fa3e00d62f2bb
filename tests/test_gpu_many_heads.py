"""Layers with more than 8 KV heads.

A work item finds its KV head from the launch parameters: for up to 8 KV
heads from per-head cumulative item counts held in the parameters, for more
by walking the heads' records.  These cases take the second path with the
needle construction of test_gpu_needles (each (batch row, live head) pair's
output must be the plain mean of its needle rows, which sit at every 64-row
quantum of the middle, at tile edges, at the sink and window rows and at a
step's appended and leaving tokens), so a lost or doubled row, or an item
attributed to the wrong head, shows: 16 and 12 KV heads with dead heads and
kept widths from 8 to 128, in plans of more than one round of workgroups
(bulk and tail items, and for a low-bit middle the full-width items
dispatched first) and of one round, and at the most KV heads a plan holds
(64: their records fill the launch parameters).
"""

import pytest

from tests.test_gpu_needles import run_case

pytestmark = pytest.mark.gpu

COUNTS16 = [32, 0, 64, 32, 0, 96, 32, 128, 8, 0, 32, 64, 0, 32, 16, 40]
COUNTS12 = [32, 64, 0, 32, 24, 0, 32, 128, 0, 48, 32, 8]
# at most 32 channels: with a 4-bit middle at batch 32 the plan dispatches
# every row's full-width items first
NARROW16 = [32, 0, 32, 16, 0, 32, 32, 8, 24, 0, 32, 32, 0, 32, 16, 8]


@pytest.mark.parametrize("step", [False, True], ids=["decode", "step"])
def test_needles_16_kv_heads_multi_round(step):
    run_case(16, 32, COUNTS16, 64, 512, 4096, step, 0, False, seed=51 + step, per_pair=24)


def test_needles_16_kv_heads_4bit_step():
    run_case(16, 32, COUNTS16, 64, 512, 4096, True, 4, False, seed=53, per_pair=24)


def test_needles_16_kv_heads_4bit_full_width_first():
    run_case(32, 32, NARROW16, 64, 512, 4096, True, 4, False, seed=59, per_pair=16)


def test_needles_12_kv_heads_paged_step():
    run_case(8, 12, COUNTS12, 32, 256, 3000, True, 0, True, seed=55, per_pair=32)


def test_needles_16_kv_heads_one_round():
    run_case(1, 16, COUNTS16, 64, 1024, 32768, True, 0, False, seed=57, oracle_pairs=1)


# the most KV heads a plan holds (LEANK_MAX_KV_HEADS): every fifth head dead,
# the others keeping 8 to 128 channels
COUNTS64 = [8 * ((7 * h) % 17) if h % 5 else 0 for h in range(64)]


def test_needles_64_kv_heads_step():
    run_case(2, 128, COUNTS64, 16, 128, 2000, True, 0, False, seed=61, per_pair=16)


def test_needles_64_kv_heads_8_query_heads_each():
    run_case(1, 512, COUNTS64, 16, 128, 2000, False, 0, False, seed=63, per_pair=16)


def test_needles_64_kv_heads_4bit_step():
    run_case(2, 64, COUNTS64, 16, 128, 2000, True, 4, False, seed=65, per_pair=16)
