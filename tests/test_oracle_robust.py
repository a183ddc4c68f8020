"""Pins for the oracle's outlier-robust calibration (oracle/transform.py robust_eig and
calibrate_tensor(rows=...)).

The ablation study ("Ablation, Statistical Inference, and Validation for KV-Cache Compression",
performance in specific regimes) reports the sample covariance corrupted by outliers on
heavy-tailed (Student-t) rows, with the calibrated eigenbasis shifting; the estimator pinned
here (spatial-sign directions, median-based variances) is the reading written in robust_eig's
docstring.  Its outputs are fixed by: a hand-computed example and its rotation, the median of
chi-squared(1) from the error function, invariance to per-row scales, the reduction to the
plain eigenbasis for rows of equal norm, consistency on Gaussian rows, and a smaller basis
error than the sample second moment on Student-t(3) rows.
"""
import math

import numpy as np
import pytest

from oracle import calibrate as OC
from oracle import allocation as OA
from oracle import transform as T


def test_chi2_1_median_from_the_error_function():
    # P(chi2_1 <= m) = P(|Z| <= sqrt(m)) = erf(sqrt(m / 2)) = 1/2
    m = T.CHI2_1_MEDIAN
    assert abs(math.erf(math.sqrt(m / 2.0)) - 0.5) < 1e-15
    assert abs(m - 0.454936423119572) < 1e-14


def test_hand_example_and_its_rotation():
    # rows (2,0), (-2,0), (2,0), (0,1): spatial-sign moment diag(3/4, 1/4) -> directions e1, e2;
    # squared projections on e1: 4, 4, 4, 0 -> median 4; on e2: 0, 0, 0, 1 -> median 0
    Y = np.array([[2.0, 0.0], [-2.0, 0.0], [2.0, 0.0], [0.0, 1.0]])
    lam, V = T.robust_eig(Y)
    np.testing.assert_allclose(lam, [4.0 / T.CHI2_1_MEDIAN, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(V, np.eye(2), atol=1e-15)
    # the same rows rotated by 30 degrees: the directions rotate with them (columns of R,
    # canonical signs), the variances do not change
    a = math.radians(30.0)
    R = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
    lam2, V2 = T.robust_eig(Y @ R.T)
    np.testing.assert_allclose(lam2, lam, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(V2, T.canonical_signs(R), atol=1e-14)


def test_per_row_scales_leave_the_directions_unchanged():
    rng = np.random.default_rng(21)
    A = rng.standard_normal((6, 6))
    Y = rng.standard_normal((500, 6)) @ A
    r = np.exp(rng.standard_normal(500) * 2.0)          # wildly different row scales
    lam, V = T.robust_eig(Y)
    lam_r, V_r = T.robust_eig(Y * r[:, None])
    np.testing.assert_allclose(np.abs(np.sum(V * V_r, axis=0)), 1.0, atol=1e-10)
    # one common scale c multiplies every variance by c^2
    lam_c, V_c = T.robust_eig(3.0 * Y)
    np.testing.assert_allclose(lam_c, 9.0 * lam, rtol=1e-12)
    np.testing.assert_allclose(V_c, V, atol=1e-12)


def test_rows_of_equal_norm_give_the_plain_eigenbasis():
    # with |y| = c for every row, S = (Y^T Y / n) / c^2: the directions are the eigenvectors of
    # the sample second moment
    rng = np.random.default_rng(22)
    Y = rng.standard_normal((400, 5)) @ np.diag([3.0, 2.0, 1.5, 1.0, 0.5])
    Y /= np.linalg.norm(Y, axis=1, keepdims=True)
    _, V = T.robust_eig(Y)
    _, Vg = T.g_weighted_eig(Y.T @ Y / Y.shape[0], np.eye(5))
    # same set of directions (robust_eig orders them by its own variances)
    overlap = np.abs(V.T @ Vg)
    np.testing.assert_allclose(np.sort(overlap.max(axis=1)), 1.0, atol=1e-10)


def _rotation(m, rng):
    q, r = np.linalg.qr(rng.standard_normal((m, m)))
    return q * np.sign(np.diag(r))[None, :]


def test_consistent_on_gaussian_rows():
    rng = np.random.default_rng(23)
    lam_true = np.array([4.0, 2.0, 1.0, 0.5])
    Q = _rotation(4, rng)
    Y = rng.standard_normal((200_000, 4)) * np.sqrt(lam_true) @ Q.T
    lam, V = T.robust_eig(Y)
    np.testing.assert_allclose(lam, lam_true, rtol=0.02)
    assert np.all(np.abs(np.sum(V * Q, axis=0)) > 0.999)


def _subspace_error(V, Q, k):
    # squared sine sum between the leading k directions of V and of Q
    P = V[:, :k].T @ Q[:, :k]
    return k - float(np.sum(P * P))


def test_heavy_tails_basis_closer_than_the_sample_second_moment():
    # Student-t(3) rows: Gaussian rows times sqrt(3 / chi2_3) per row
    rng = np.random.default_rng(24)
    m, n, k = 16, 3000, 4
    lam_true = 1.0 / np.arange(1, m + 1) ** 1.2
    Q = _rotation(m, rng)
    z = rng.standard_normal((n, m)) * np.sqrt(lam_true) @ Q.T
    Y = z * np.sqrt(3.0 / rng.chisquare(3, size=n))[:, None]
    _, V_rob = T.robust_eig(Y)
    _, V_smp = T.g_weighted_eig(Y.T @ Y / n, np.eye(m))
    e_rob, e_smp = _subspace_error(V_rob, Q, k), _subspace_error(V_smp, Q, k)
    assert e_rob < 0.5 * e_smp, (e_rob, e_smp)
    # the variances keep the true ratios up to one common factor
    lam_rob, _ = T.robust_eig(Y)
    ratio = lam_rob[:k] / lam_true[:k]
    assert ratio.max() / ratio.min() < 1.25


def test_zero_rows_count_in_the_medians_only():
    Y = np.array([[2.0, 0.0], [-2.0, 0.0], [2.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    lam, V = T.robust_eig(Y)
    # spatial-sign moment over the four non-zero rows: unchanged directions; squared
    # projections on e1: 4, 4, 4, 0, 0 -> median 4
    np.testing.assert_allclose(V, np.eye(2), atol=1e-15)
    np.testing.assert_allclose(lam, [4.0 / T.CHI2_1_MEDIAN, 0.0], atol=1e-15)
    lam0, V0 = T.robust_eig(np.zeros((3, 2)))
    np.testing.assert_array_equal(lam0, [0.0, 0.0])


@pytest.mark.parametrize("n_seg", [1, 2])
def test_calibrate_with_rows_uses_the_robust_pairs(n_seg):
    rng = np.random.default_rng(25)
    d, n_kv, dh, r, g = 24, 2, 8, 8, 2
    W = rng.standard_normal((d, n_kv * dh))
    X = rng.standard_normal((300, d)) * np.sqrt(3.0 / rng.chisquare(3, size=300))[:, None]
    out = OC.calibrate_tensor(None, W, n_seg, r, g, 3.0, rows=X, robust=True)
    seg_cols = n_kv * dh // n_seg
    R = int(math.floor(3.0 * seg_cols + 1e-9))
    for s in range(n_seg):
        Ws = W[:, s * seg_cols:(s + 1) * seg_cols]
        lam, V = T.robust_eig(X @ Ws)
        w, _ = OA.water_fill(OA.group_variances(lam[:r], g), g, R, 16, 8)
        np.testing.assert_array_equal(out["widths"][s], w)
        np.testing.assert_allclose(out["sigma2"][s], lam[:r], rtol=1e-12)
