"""Pins for oracle.allocation: reverse water-filling (CPU only)."""
import itertools
import math

import numpy as np
import pytest

from oracle import allocation as A


def _profiles():
    rng = np.random.default_rng(11)
    for n in (1, 3, 8, 32):
        yield np.sort(rng.lognormal(0, 2, n))[::-1]
        yield (np.arange(1, n + 1) ** -1.2)[::1] * 7
    yield np.full(6, 2.5)


@pytest.mark.parametrize("g,scale_bits", [(1, 0), (4, 16), (16, 16)])
def test_budget_met_and_next_step_exceeds(g, scale_bits):
    for v in _profiles():
        for R in (0, 17, 100, 640, 5000):
            w, th = A.water_fill(v, g, R, scale_bits)
            assert A.cost(w, g, scale_bits) <= R
            nxt = [t for t in A.breakpoints(v) if t < th]
            if nxt:
                t2 = max(nxt)
                w2 = np.array([np.sum(v[k] * 4.0 ** -(np.arange(1, 9) - 0.5) >= t2) for k in range(v.size)])
                assert A.cost(w2, g, scale_bits) > R


def test_widths_track_half_log2():
    # (2): 0 < b < 8 -> |b - 1/2 log2(v/theta)| <= 1/2 ; b = 0 -> 1/2 log2(v/theta) < 1/2
    for v in _profiles():
        for R in (40, 300, 2000):
            w, th = A.water_fill(v, 4, R, 16)
            if math.isinf(th):
                assert np.all(w == 0)
                continue
            rate = 0.5 * np.log2(v / th)
            mid = (w > 0) & (w < 8)
            assert np.all(np.abs(w[mid] - rate[mid]) <= 0.5 + 1e-12)
            assert np.all(rate[w == 0] < 0.5 + 1e-12)


def test_textbook_two_components():
    # Continuous reverse water-filling with variances (4, 1) and a 1-bit total gives water
    # level theta = 1 and rates (1/2 log2(4/1), 0) = (1, 0).
    v = np.array([4.0, 1.0])
    w, th = A.water_fill(v, 1, 1, 0)
    assert w.tolist() == [1, 0]
    assert A.widths_at(v, 1.0).tolist() == [1, 0]
    # and with 3 bits: continuous theta solves 1/2log2(4/t)+1/2log2(1/t) = 3 -> t = 1/4,
    # rates (2, 1), integers, so the rounding reading must return them
    w3, _ = A.water_fill(v, 1, 3, 0)
    assert w3.tolist() == [2, 1]
    assert A.widths_at(v, 0.25).tolist() == [2, 1]


def test_equal_variances_give_uniform_widths():
    v = np.full(8, 3.0)
    for R in range(0, 8 * (16 * 8 + 16) + 1, 37):
        w, _ = A.water_fill(v, 16, R, 16)
        assert len(set(w.tolist())) == 1


def test_nonincreasing_for_sorted_variances():
    for v in _profiles():
        w, _ = A.water_fill(v, 16, 1500, 16)
        assert np.all(np.diff(w) <= 0)


def test_brute_force_over_all_water_levels():
    # Enumerate every candidate level (all breakpoints and +inf) without assuming the cost is
    # monotone; the scan must pick the smallest level whose widths fit.
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 5))
        v = rng.lognormal(0, 1.5, n)
        g = int(rng.choice([1, 2, 4]))
        sb = int(rng.choice([0, 16]))
        R = int(rng.integers(0, n * (8 * g + sb) + 2))
        best_t, best_w = math.inf, np.zeros(n, dtype=int)
        for t in A.breakpoints(v):
            w = np.array([sum(1 for j in range(1, 9) if v[k] * 4.0 ** -(j - 0.5) >= t) for k in range(n)])
            if A.cost(w, g, sb) <= R and t < best_t:
                best_t, best_w = t, w
        w, th = A.water_fill(v, g, R, sb)
        assert w.tolist() == best_w.tolist()
        assert th == best_t


def test_group_variance_is_mean():
    assert A.group_variances(np.array([4.0, 2.0, 1.0, 3.0]), 2).tolist() == [3.0, 2.0]


def test_zero_bit_groups_are_dropped():
    assert A.active_groups(np.array([3, 0, 2, 0])) == [0, 2]
