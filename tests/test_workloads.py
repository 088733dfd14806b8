"""Seeded input generators: determinism, rounding and the stated recipe."""
import numpy as np
import pytest
import torch

from recurrent_sequence_mixer_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000) * 10 ** rng.uniform(-30, 30, 100000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.0078125, 3.4e38, 1e-40]])
    ours = W.round_bf16(a)
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_generate_is_deterministic_and_rounded():
    wl = W.WORKLOADS[1].replace(B=2, H=2, T=70)
    a, b = W.generate(wl), W.generate(wl)
    assert W.sha256(a) == W.sha256(b)
    for name in ("q", "k", "v"):
        x = a[name]
        np.testing.assert_array_equal(W.round_bf16(x), x)  # bf16-representable
    np.testing.assert_allclose(np.linalg.norm(a["q"].astype(np.float64), axis=-1), 1, atol=1e-2)
    assert a["eta"].dtype == np.float32 and np.all((a["eta"] > 0) & (a["eta"] < 1))
    assert a["alpha"].shape == (2, 2, 70)
    assert abs(a["S0"].std() - 0.1) < 0.01


def test_generate_variants():
    pg = W.generate(W.WORKLOADS[2].replace(B=1, H=3, T=40))
    np.testing.assert_allclose(np.linalg.norm(pg["k"].astype(np.float64), axis=-1), 1, atol=1e-2)
    assert pg["mu_log"].shape == (3,) and pg["alphaP"].shape == (1, 3, 40)
    kd = W.generate(W.WORKLOADS[3].replace(B=1, H=2, T=40))
    assert kd["alpha"].shape == (1, 2, 40, 128) and kd["omega"].shape == (1, 2, 40, 128)
    np.testing.assert_array_equal(W.round_bf16(kd["alpha"]), kd["alpha"])
    assert np.all(kd["r"] > 0) and np.all(kd["omega"] > 0)
    z = W.generate(W.WORKLOADS[0])
    assert np.all(z["S0"] == 0) and z["q"].shape == (1, 1, 256, 64)


def test_decode_steps_independent_streams():
    wl = W.WORKLOADS[4]
    small = W.DecodeWorkload("t", 4, 2, 8, 8, 3)
    s1 = W.generate_decode_step(small, 1)
    s1b = W.generate_decode_step(small, 1)
    s2 = W.generate_decode_step(small, 2)
    assert W.sha256(s1) == W.sha256(s1b) and W.sha256(s1) != W.sha256(s2)
    assert wl.N == 512 and wl.steps == 256


def test_pgdn_centre_spread_per_head():
    """mu_spread gives every head its own PGDN centre, symmetric about mu_log;
    without it all heads share mu_log (the draws are unchanged either way)."""
    base = W.WORKLOADS[2].replace(B=1, H=4, T=8)
    a = W.generate(base)
    b = W.generate(base.replace(mu_spread=0.75))
    np.testing.assert_array_equal(a["mu_log"], np.float32(np.log(4.0)))
    assert len(set(b["mu_log"].tolist())) == 4
    np.testing.assert_allclose(b["mu_log"].mean(), np.log(4.0), rtol=1e-6)
    np.testing.assert_allclose(b["mu_log"].max() - b["mu_log"].min(), 1.5, rtol=1e-6)
    for name in ("q", "k", "v", "eta", "alpha", "alphaP", "betaP", "S0"):
        np.testing.assert_array_equal(a[name], b[name])


def test_alpha_mean_sets_decay_strength():
    """alpha_mean moves the decay distribution; the other draws are unchanged."""
    base = W.WORKLOADS[3].replace(B=1, H=2, T=64)
    a = W.generate(base)
    b = W.generate(base.replace(alpha_mean=-1.0))
    assert np.median(np.log2(b["alpha"].astype(np.float64))) < -1.5 < np.median(np.log2(a["alpha"].astype(np.float64)))
    for name in ("q", "k", "v", "omega", "r", "S0"):
        np.testing.assert_array_equal(a[name], b[name])
