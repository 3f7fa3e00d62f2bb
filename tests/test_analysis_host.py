"""Host analysis helpers of the library against the CPU oracle (no GPU needed)."""

import numpy as np
import pytest

import decode_attention_channel_amd as dac
import oracle
from synthetic import CONFIGS, alpha_for, get_config


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_retention_and_hf_ratio_match_oracle(cfg):
    alpha = alpha_for(cfg)
    mask, _, _ = oracle.build_mask(alpha, cfg.prune_pct, cfg.align)
    np.testing.assert_allclose(dac.leank_pair_retention(mask), oracle.pair_retention(mask),
                               rtol=0, atol=1e-12)
    for n_hf in (0, 1, 16, 32, 64):
        np.testing.assert_allclose(dac.leank_head_hf_ratio(alpha, n_hf),
                                   oracle.head_hf_ratio(alpha, n_hf), rtol=1e-12, atol=1e-15)


def test_synthetic_alpha_keeps_low_frequency_pairs_more():
    # the recipe's f_c rises with the pair index, so retention should too
    cfg = get_config("llama32_b64_gen")
    mask, _, _ = oracle.build_mask(alpha_for(cfg), cfg.prune_pct, cfg.align)
    ret = dac.leank_pair_retention(mask)
    assert ret[:16].mean() < ret[48:].mean()


def test_rank_correlation_matches_oracle():
    rng = np.random.default_rng(3)
    for cfg in (get_config("tiny"), get_config("llama_b64_4k"), get_config("qwen_b16_32k")):
        a = alpha_for(cfg)
        b = alpha_for(cfg, seed=cfg.alpha_seed + 1)
        for x, y in ((a, b), (a, a * 1.5 + 0.1), (np.round(a, 1), np.round(b, 1))):
            got = dac.leank_rank_correlation(x, y)
            ref = oracle.rank_correlation(x.astype(np.float32), y.astype(np.float32))
            np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)
    x = rng.standard_normal(1000).astype(np.float32)
    assert dac.leank_rank_correlation(x, -x)[1] == pytest.approx(-1.0, abs=1e-12)


def test_analysis_rejects_bad_input():
    with pytest.raises(dac.LeankError):
        dac.leank_rank_correlation(np.array([1.0, np.nan]), np.array([1.0, 2.0]))
    with pytest.raises(dac.LeankError):
        dac.leank_head_hf_ratio(np.ones((1, 1, 8), np.float32), 5)
    with pytest.raises(dac.LeankError):
        dac.leank_rank_correlation(np.array([1.0]), np.array([1.0]))
