"""Pins for oracle.transform: G-weighted SVD, energy rank (CPU only)."""
import numpy as np
import pytest

from oracle import transform, calibrate
from synth import TINY, generators as gen


def _tiny_calib():
    Q = gen.basis(TINY)
    h = gen.hidden_rows(TINY, TINY.calib_rows, gen.STREAM_CALIB, Q)
    wk, wv, wq, wo = gen.projection_weights(TINY)
    return h, wk, wv


def test_latent_decorrelated_and_variance_sorted():
    # (1): on the calibration rows the latent's second moment is diag(sigma^2), descending.
    h, wk, _ = _tiny_calib()
    G = transform.gram(h)
    lam, V = transform.g_weighted_eig(G, wk)
    r = 16
    c = h @ (wk @ V[:, :r])
    M = c.T @ c / h.shape[0]
    scale = lam[0]
    assert np.abs(M - np.diag(lam[:r])).max() < 1e-10 * scale
    assert np.all(np.diff(lam) <= 0)
    # marginal variances of the latent coordinates are the eigenvalues
    assert np.allclose(np.mean(c ** 2, axis=0), lam[:r], rtol=1e-10)


def test_eckart_young_truncation_error():
    # E||hW - hW V_r V_r^T||^2 = sum of discarded eigenvalues
    h, wk, _ = _tiny_calib()
    G = transform.gram(h)
    lam, V = transform.g_weighted_eig(G, wk)
    for r in (4, 16, 40):
        k = h @ wk
        err = np.mean(np.sum((k - k @ V[:, :r] @ V[:, :r].T) ** 2, axis=1))
        assert err == pytest.approx(lam[r:].sum(), rel=1e-9)


def test_g_weighting_beats_weight_space_truncation():
    # The activation-metric error of the G-weighted basis is minimal over rank-r projections,
    # so it is never worse than truncating the plain SVD of W (weight space).
    h, wk, _ = _tiny_calib()
    G = transform.gram(h)
    lam, V = transform.g_weighted_eig(G, wk)
    _, _, Vt = np.linalg.svd(wk, full_matrices=False)
    k = h @ wk
    for r in (4, 8, 16):
        e_g = np.mean(np.sum((k - k @ V[:, :r] @ V[:, :r].T) ** 2, axis=1))
        Vw = Vt[:r].T
        e_w = np.mean(np.sum((k - k @ Vw @ Vw.T) ** 2, axis=1))
        assert e_g <= e_w * (1 + 1e-12)
        assert e_g < e_w  # strict on this correlated input


def test_identity_gram_gives_svd_of_w():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((24, 10))
    lam, V = transform.g_weighted_eig(np.eye(24), W)
    _, s, Vt = np.linalg.svd(W, full_matrices=False)
    assert np.allclose(lam, s ** 2, rtol=1e-12)
    # same vectors up to sign
    assert np.allclose(np.abs(V.T @ Vt.T), np.eye(10), atol=1e-10)


def test_identity_weights_give_pca_of_gram():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((200, 12)) @ rng.standard_normal((12, 12))
    G = transform.gram(X)
    lam, V = transform.g_weighted_eig(G, np.eye(12))
    U, s, _ = np.linalg.svd(G)
    assert np.allclose(lam, s, rtol=1e-11)
    assert np.allclose(np.abs(V.T @ U), np.eye(12), atol=1e-9)


def test_gram_is_uncentred_second_moment():
    rows = np.array([[1.0, 2.0], [3.0, -1.0]])
    # E[h^T h] = ([1,2]^T[1,2] + [3,-1]^T[3,-1]) / 2
    assert np.array_equal(transform.gram(rows), np.array([[5.0, -0.5], [-0.5, 2.5]]))


def test_canonical_sign_rule():
    v = np.array([[0.1, -0.6], [-0.9, 0.6], [0.2, 0.1]])
    c = transform.canonical_signs(v)
    assert c[1, 0] == 0.9          # largest magnitude made positive
    assert c[0, 1] == 0.6          # tie between rows 0 and 1 -> first index positive


def test_energy_rank():
    lam = np.array([5.0, 3.0, 1.0, 1.0])
    assert transform.energy_rank(lam, 0.5) == 1
    assert transform.energy_rank(lam, 0.8) == 2
    assert transform.energy_rank(lam, 0.81) == 3
    assert transform.energy_rank(lam, 1.0) == 4


def test_w_up_rows_orthonormal_and_w_down_is_w_times_w_up_t():
    h, wk, wv = _tiny_calib()
    G = transform.gram(h)
    out = calibrate.calibrate(G, wk, wv, 1, 16, 4, 2.0)
    for t, W in (("k", wk), ("v", wv)):
        up = out[t]["w_up"]
        assert np.allclose(up @ up.T, np.eye(up.shape[0]), atol=1e-12)
        assert np.allclose(out[t]["w_down"], W @ up.T, atol=1e-12)


def test_gap_rank_finds_a_planted_gap_and_leaves_smooth_spectra():
    # a drop of 7000x after the 4th eigenvalue is the largest ratio: trimmed to 4 when the
    # threshold is below it, kept whole above it
    lam = np.array([10.0, 9.0, 8.0, 7.0, 1e-3, 9e-4, 8e-4, 7e-4, 6e-4, 5e-4])
    assert transform.gap_rank(lam, 8, 10.0) == 4
    assert transform.gap_rank(lam, 8, 1e5) == 8
    # the gap must lie inside the leading r_max eigenvalues
    assert transform.gap_rank(lam, 4, 10.0) == 4 and transform.gap_rank(lam, 3, 1.01) == 2   # 9/8 > 10/9
    # geometric decay (every ratio 1/0.9) and a flat spectrum have no gap worth trimming
    geo = 0.9 ** np.arange(40)
    assert transform.gap_rank(geo, 32, 2.0) == 32
    assert transform.gap_rank(np.ones(20), 16, 1.5) == 16
    # ties: the first largest ratio wins
    assert transform.gap_rank(np.array([8.0, 4.0, 2.0, 1.0]), 4, 1.5) == 1


def test_gap_rank_recovers_the_rank_of_a_rank_deficient_weight():
    # W of rank 5: M = W^T G W has 5 positive eigenvalues and round-off after them
    rng = np.random.default_rng(9)
    W = rng.standard_normal((40, 5)) @ rng.standard_normal((5, 24))
    G = transform.gram(rng.standard_normal((500, 40)))
    lam, _ = transform.g_weighted_eig(G, W)
    assert transform.gap_rank(lam, 16, 1e6) == 5
    assert transform.energy_rank(lam, 1 - 1e-12) == 5


def test_encode_latent_of_calibration_rows_is_diagonal():
    # attention.encode_latent with calibrate's W_down (x W_down, W_down [d_model x r_act]) on the
    # calibration rows: second moment diag(sigma^2) of the active columns, K columns then V
    # columns.  A transposed operand or the wrong tensor's columns breaks the diagonal.
    from oracle import attention as OA
    h, wk, wv = _tiny_calib()
    G = transform.gram(h)
    cal = calibrate.calibrate(G, wk, wv, 1, 16, 4, TINY.budget_bits)
    c = OA.encode_latent(h, cal["w_down"])
    rk = cal["k"]["w_down"].shape[1]
    for cols, part in ((slice(0, rk), cal["k"]), (slice(rk, None), cal["v"])):
        cc = c[:, cols]
        M = cc.T @ cc / h.shape[0]
        act = [k for k, b in enumerate(part["widths"][0]) if b > 0]
        s2 = np.concatenate([part["sigma2"][0][4 * k:4 * k + 4] for k in act])
        assert np.abs(M - np.diag(s2)).max() < 1e-10 * s2[0]
