"""Pins for the oracle's rank rules in calibration (CPU only).

The energy rule keeps the smallest rank holding a target share of the energy ([SPECTRAL-KV]
Technical principle 1); the gap rule trims at a spectral gap (a reading of the ablation study's
d_eff criterion, Core contributions 3).  Either way the kept rank is rounded up to whole groups,
later groups get no bits, and the budget is water-filled over the groups kept.
"""
import numpy as np
import pytest

from oracle import calibrate as OC, transform


def _planted(d=64, n=64, k=24, seed=2):
    """W = Q diag(sqrt(lam)) P^T with G = I: the eigenvalues of W^T G W are exactly lam
    (k values from 10 down to 5, then a 50-fold drop to a tail holding about 1.6 % of the
    energy)."""
    rng = np.random.default_rng(seed)
    lam = np.concatenate([np.linspace(10.0, 5.0, k), np.linspace(0.1, 0.05, n - k)])
    Q = np.linalg.qr(rng.standard_normal((d, d)))[0][:, :n]
    P = np.linalg.qr(rng.standard_normal((n, n)))[0]
    return np.eye(d), Q @ np.diag(np.sqrt(lam)) @ P.T, lam


def test_planted_spectrum_is_recovered():
    G, W, lam = _planted()
    got, _ = transform.g_weighted_eig(G, W)
    assert np.allclose(got, np.sort(lam)[::-1], rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("rule,kw", [("energy", dict(energy=0.98)), ("gap", dict(gap_ratio=20.0))])
def test_rules_cap_at_the_planted_rank(rule, kw):
    G, W, lam = _planted(k=24)
    g = 16
    cut = OC.calibrate_tensor(G, W, 1, 48, g, 3.0, rank_rule=rule, **kw)
    full = OC.calibrate_tensor(G, W, 1, 48, g, 3.0)
    w = cut["widths"][0]
    assert np.all(w[2:] == 0) and np.all(w[:2] > 0)          # ceil(24 / 16) = 2 groups kept
    assert np.any(full["widths"][0][2:] > 0)                   # the fixed rule spends bits past them
    # the budget concentrates: each kept group has at least the width it had before
    assert np.all(w[:2] >= full["widths"][0][:2])
    assert cut["w_up"].shape[0] == 16 * int((w > 0).sum())
    assert cut["energy_rank"][0] == (24 if rule == "energy" else -1)


def test_rules_reduce_to_the_fixed_rule_when_nothing_is_trimmed():
    rng = np.random.default_rng(4)
    d, n = 48, 32
    G = transform.gram(rng.standard_normal((600, d)) * (0.97 ** np.arange(d)))
    W = rng.standard_normal((d, n))
    base = OC.calibrate_tensor(G, W, 1, 24, 8, 2.0)
    for rule, kw in (("energy", dict(energy=1.0)), ("gap", dict(gap_ratio=1e9))):
        c = OC.calibrate_tensor(G, W, 1, 24, 8, 2.0, rank_rule=rule, **kw)
        assert np.array_equal(c["widths"], base["widths"])
        assert np.allclose(c["w_down"], base["w_down"])


def test_fixed_width_with_a_rank_rule():
    G, W, lam = _planted(k=20)
    c = OC.calibrate_tensor(G, W, 1, 64, 8, 0.0, fixed_width=3, rank_rule="gap", gap_ratio=20.0)
    assert c["widths"][0].tolist() == [3, 3, 3] + [0] * 5      # ceil(20 / 8) = 3 groups
