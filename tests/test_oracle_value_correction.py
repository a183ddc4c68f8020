"""Pins for the oracle's value-latent correction (oracle/calibrate.py value_correction).

Stage 1 of the SPECTRA pipeline folds a closed-form correction of W_O into the weights without
giving a formula; the reading pinned here is the least-squares map F from the calibration
rows' dequantised value latents to their exact latents, folded into W_up_V.  Pinned by a
closed form (group size 1, latents that are powers of two: the quantiser reconstructs every
value as (1 - 2^-b) c, so F = diag(2^b / (2^b - 1)) whatever the correlations), by
optimality on the calibration rows (never worse than no correction), and by F tending to the
identity as the bits grow.
"""
import numpy as np
import pytest

from oracle import calibrate as OC
from oracle import quant as OQ


@pytest.mark.parametrize("widths", [[1], [2], [3], [1, 2, 3, 8]])
def test_closed_form_for_exactly_scaled_latents(widths):
    rng = np.random.default_rng(41)
    r = len(widths)
    # latents +-2^k with correlated signs across columns; W_down = I so C = rows
    n = 64
    C = (2.0 ** rng.integers(-6, 6, size=(n, r))) * np.where(rng.random((n, 1)) < 0.5, -1.0, 1.0)
    C[:, 1:] *= np.where(rng.random((n, r - 1)) < 0.8, 1.0, -1.0) if r > 1 else 1.0
    F = OC.value_correction(C, np.eye(r), widths, 1)
    expect = np.diag([2.0 ** b / (2.0 ** b - 1.0) for b in widths])
    np.testing.assert_allclose(F, expect, rtol=1e-12, atol=1e-12)
    # the premise: every dequantised value is (1 - 2^-b) c
    u, s = OQ.quantize_latent(C.astype(np.float32), widths, 1)
    Ch = OQ.dequantize_latent(u, s, widths, 1)
    np.testing.assert_array_equal(Ch, C * (1.0 - 2.0 ** -np.array(widths, dtype=np.float64)))


def _rows(rng, n, d):
    lam = np.arange(1, d + 1) ** -1.0
    return rng.standard_normal((n, d)) * np.sqrt(lam)


@pytest.mark.parametrize("g,widths", [(2, [3, 2, 1]), (4, [4, 2])])
def test_never_worse_than_no_correction_on_the_calibration_rows(g, widths):
    rng = np.random.default_rng(42)
    d = 16
    r = g * len(widths)
    X = _rows(rng, 4000, d)
    Wd = rng.standard_normal((d, r)) / 4.0
    F = OC.value_correction(X, Wd, widths, g)
    C = X @ Wd
    u, s = OQ.quantize_latent(C.astype(np.float32), widths, g)
    Ch = OQ.dequantize_latent(u, s, widths, g)
    e0 = np.sum((Ch - C) ** 2)
    e1 = np.sum((Ch @ F - C) ** 2)
    assert e1 <= e0
    assert e1 < 0.99 * e0                               # and a real gain at these widths
    # a transposed F is not the optimum (the fit is not symmetric)
    assert np.sum((Ch @ F.T - C) ** 2) > e1


def test_tends_to_identity_with_more_bits():
    rng = np.random.default_rng(43)
    d, g = 12, 4
    X = _rows(rng, 6000, d)
    Wd = rng.standard_normal((d, 8)) / 3.0
    dev = [np.abs(OC.value_correction(X, Wd, [b, b], g) - np.eye(8)).max() for b in (1, 2, 4, 8)]
    assert all(a > b for a, b in zip(dev, dev[1:])), dev
    assert dev[-1] < 1e-2
