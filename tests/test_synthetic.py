"""Statistics of the seeded synthetic workloads (CPU only)."""

import math

import numpy as np
import pytest
import torch

from synthetic import (CONFIGS, custom_config, firing_law, make_layer, make_tokens,
                       rank_probabilities, solve_exponent)


def _hot_fraction(f, share=0.8):
    f = np.sort(f)[::-1]
    cs = np.cumsum(f)
    return (np.searchsorted(cs, share * cs[-1]) + 1) / len(f)


@pytest.mark.parametrize("key,hot", [("c2", 0.17), ("c3", 0.26), ("c5", 0.17)])
def test_power_law_matches_the_pages_hot_share(key, hot):
    # 17% (OPT-30B) and 26% (LLaMA2-ReGLU-70B) of neurons carry 80% of activations
    cfg = CONFIGS[key]
    f = rank_probabilities(cfg)
    assert abs(f.mean() - cfg.mean) < 1e-6
    assert abs(_hot_fraction(f) - hot) < 2e-3
    assert np.all(np.diff(f) <= 0) and f.min() >= 1e-4 and f.max() <= 0.999


def test_solved_exponents():
    assert abs(solve_exponent(28672, 0.10, 0.17) - 1.566) < 2e-3
    assert abs(solve_exponent(28672, 0.20, 0.26) - 1.675) < 2e-3


def test_zipf_configs():
    for key in ("c1", "c4"):
        cfg = CONFIGS[key]
        f = rank_probabilities(cfg)
        assert abs(f.mean() - cfg.mean) < 1e-6
        ratio = f[9] / f[19]
        assert ratio == pytest.approx(2 ** 1.1, rel=1e-9) or f[9] >= 0.999


def test_layer_shapes_norms_and_bias():
    cfg = custom_config("reglu", d=96, ffn=200, r=24, mean=0.15)
    L = make_layer(cfg)
    for k in ("W_up", "W_gate", "W_down"):
        assert L[k].shape == (200, 96) and L[k].dtype == torch.float16
        n = torch.linalg.vector_norm(L[k].float(), dim=1)
        assert torch.all((n - 1).abs() < 2e-3)
    assert L["P1"].shape == (24, 96) and L["P2"].shape == (200, 24)
    assert L["b_up"] is None and L["b_gate"].dtype == torch.float32
    from scipy.special import ndtri
    np.testing.assert_allclose(L["b_gate"].numpy(), ndtri(L["f"]).astype(np.float32))
    # the rank permutation scatters probabilities over neurons
    assert not np.all(np.diff(L["f"]) <= 0)
    assert abs(L["f"].mean() - 0.15) < 1e-6


def test_seeded_and_distinct_per_layer():
    cfg = custom_config("relu", d=64, ffn=128, r=8)
    a, b, c = make_layer(cfg, 0), make_layer(cfg, 0), make_layer(cfg, 1)
    assert torch.equal(a["W_up"], b["W_up"]) and torch.equal(a["P2"], b["P2"])
    assert not torch.equal(a["W_up"], c["W_up"])
    t1, t2 = make_tokens(cfg, 4), make_tokens(cfg, 4)
    assert torch.equal(t1, t2) and t1.dtype == torch.float16


def test_predictor_rate_is_calibrated():
    """Predicted active fraction ~= mean firing probability (approximate calibration)."""
    cfg = custom_config("relu", d=512, ffn=2048, r=64, mean=0.10)
    L = make_layer(cfg)
    X = make_tokens(cfg, 256).float()
    h = torch.relu(X @ L["P1"].float().T)
    z = h @ L["P2"].float().T + L["b2"]
    rate = (z > 0).float().mean().item()
    assert abs(rate - 0.10) < 0.03, rate
