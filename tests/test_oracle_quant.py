"""Pins for oracle.quant: per-token group quantiser (CPU only)."""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_quant():
    d = {}
    for line in open(os.path.join(GOLDEN, "quant_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, *vals = line.split()
        d[k] = [float(x) for x in vals]
    return d


def test_hand_computed_example():
    d = _golden_quant()
    c = np.array(d["c"], dtype=np.float32)
    b = int(d["b"][0])
    u, s = quant.quantize(c[None, :], b)
    assert float(s[0]) == d["s"][0]
    assert u[0].tolist() == [int(x) for x in d["u"]]
    assert quant.dequantize(u, s, b)[0].tolist() == d["chat"]


def test_scale_rounds_half_to_even():
    one = np.float32(1.0)
    a1 = np.array([[one + np.float32(2.0 ** -11)]], dtype=np.float32)
    a2 = np.array([[one + np.float32(3 * 2.0 ** -11)]], dtype=np.float32)
    assert float(quant.scales_fp16(a1, 1)[0]) == 1.0
    assert float(quant.scales_fp16(a2, 1)[0]) == 1.0 + 2.0 ** -9


def test_fp16_overflow_saturates():
    c = np.array([[1e6, -3.0]], dtype=np.float32)
    s = quant.scales_fp16(c, 1)
    assert float(s[0]) == 65504.0


def test_zero_group_gives_zero_codes_and_values():
    for b in range(1, 9):
        u, s = quant.quantize(np.zeros((3, 4), np.float32), b)
        assert np.all(u == 0) and np.all(s == 0)
        assert np.all(quant.dequantize(u, s, b) == 0)


def _nearest_level_exact(c: float, s: float, b: int) -> int:
    """Brute force over all 2^b levels s (u - h) in exact arithmetic, ties to even u."""
    cf, sf = Fraction(c), Fraction(s)
    h = Fraction(2 ** b - 1, 2)
    best = None
    for u in range(2 ** b):
        d = abs(cf - sf * (u - h))
        if best is None or d < best[0] or (d == best[0] and u % 2 == 0):
            best = (d, u)
    return best[1]


def test_formula_equals_brute_force_nearest_level():
    rng = np.random.default_rng(7)
    n_checked = 0
    for b in range(1, 9):
        c = (rng.standard_normal((60, 4)) * rng.lognormal(0, 2, (60, 1))).astype(np.float32)
        u, s = quant.quantize(c, b)
        for i in range(c.shape[0]):
            sf = float(s[i])
            for j in range(4):
                exact = _nearest_level_exact(float(c[i, j]), sf, b)
                # the float32 formula may only differ when the exact value sits within one
                # float32 rounding of a decision boundary
                x = Fraction(float(c[i, j])) / Fraction(sf) + Fraction(2 ** b - 1, 2)
                frac = x - int(x) if x >= 0 else None
                near_tie = frac is not None and abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 20)
                if not near_tie:
                    assert u[i, j] == exact, (b, c[i, j], sf)
                    n_checked += 1
    assert n_checked > 1500


def test_reconstruction_error_bound():
    rng = np.random.default_rng(8)
    for b in range(1, 9):
        c = (rng.standard_normal((500, 16)) * 3).astype(np.float32)
        u, s = quant.quantize(c, b)
        chat = quant.dequantize(u, s, b)
        A = np.abs(c).max(axis=1).astype(np.float64)
        sd = s.astype(np.float64)
        # |c - c^| <= s/2 inside the tiled range, plus the fp16 rounding slack of the range
        slack = np.abs(A - sd * 2 ** (b - 1))
        assert np.all(np.abs(c - chat) <= (sd / 2 + slack)[:, None] + 1e-12)


def test_dequantised_value_exact_in_float32():
    rng = np.random.default_rng(9)
    for b in range(1, 9):
        with np.errstate(over="ignore"):
            s = rng.lognormal(0, 4, 2000).astype(np.float16)
        s = s[np.isfinite(s) & (s > 0)]
        u = rng.integers(0, 2 ** b, s.size)
        v64 = quant.dequantize(u[:, None], s, b)[:, 0]
        v32 = s.astype(np.float32) * (u.astype(np.float32) - np.float32((2 ** b - 1) / 2))
        assert np.array_equal(v64, v32.astype(np.float64))


def test_codes_stay_in_range_and_use_extremes():
    c = np.array([[-1.0, -0.4, 0.4, 1.0]], dtype=np.float32)
    for b in range(1, 9):
        u, _ = quant.quantize(c, b)
        assert u.min() == 0 and u.max() == 2 ** b - 1


def test_latent_helpers_split_columns_by_group():
    rng = np.random.default_rng(10)
    c = rng.standard_normal((5, 12)).astype(np.float32)
    u, s = quant.quantize_latent(c, [3, 1, 5], 4)
    for i, b in enumerate([3, 1, 5]):
        uu, ss = quant.quantize(c[:, 4 * i:4 * i + 4], b)
        assert np.array_equal(u[:, 4 * i:4 * i + 4], uu) and np.array_equal(s[:, i], ss)
    back = quant.dequantize_latent(u, s, [3, 1, 5], 4)
    assert back.shape == (5, 12)
