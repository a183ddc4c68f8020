"""Rate allocation by reverse water-filling over groups of latent coordinates (oracle).

[SPECTRA] SPECTRA pipeline, stage 2: bits are allocated by reverse water-filling on the
measured marginal variances of the latent coordinates; high-variance coordinates get more
bits, low-variance ones fewer, down to zero.  Adjacent coordinates are grouped and share one
width so that the cache stays append-only.  [SPECTRA] Methodology, second observation:
channels that receive zero bits are discarded, which merges quantisation and rank reduction.

Readings (the pages give no formula):
  * marginal variance of a group = mean of its coordinates' variances;
  * textbook reverse water-filling gives a group the rate 1/2 log2(v / theta) when v > theta;
    widths are that rate rounded to the nearest integer and clamped to [0, max_width]:
        b_k(theta) = clamp(floor(1/2 log2(v_k / theta) + 1/2), 0, max_width);
  * the budget counts code bits and the fp16 scale of every non-empty group:
        cost(theta) = sum_{b_k > 0} (g * b_k + scale_bits)  <=  R;
  * theta is lowered while the cost stays within R.  b_k steps from j-1 to j exactly at
    theta = v_k * 4^-(j - 1/2); the scan visits these breakpoints from the largest down and
    stops before the first one whose cost exceeds R.  Equal breakpoints are taken together.
"""
import math
import numpy as np


def group_variances(sigma2: np.ndarray, g: int) -> np.ndarray:
    s = np.asarray(sigma2, dtype=np.float64)
    assert s.size % g == 0
    return s.reshape(-1, g).mean(axis=1)


def widths_at(v: np.ndarray, theta: float, max_width: int = 8) -> np.ndarray:
    """b_k(theta) = clamp(floor(1/2 log2(v_k/theta) + 1/2), 0, max_width)."""
    v = np.asarray(v, dtype=np.float64)
    if math.isinf(theta):
        return np.zeros(v.size, dtype=np.int64)
    out = np.zeros(v.size, dtype=np.int64)
    pos = v > 0
    r = 0.5 * np.log2(v[pos] / theta) + 0.5
    out[pos] = np.clip(np.floor(r), 0, max_width).astype(np.int64)
    return out


def cost(widths: np.ndarray, g: int, scale_bits: int = 16) -> int:
    w = np.asarray(widths, dtype=np.int64)
    return int(np.sum(np.where(w > 0, g * w + scale_bits, 0)))


def breakpoints(v: np.ndarray, max_width: int = 8) -> np.ndarray:
    """All theta at which some width increases: v_k * 4^-(j - 1/2), j = 1..max_width."""
    v = np.asarray(v, dtype=np.float64)
    j = np.arange(1, max_width + 1, dtype=np.float64)
    bp = v[v > 0][:, None] * np.power(4.0, -(j - 0.5))[None, :]
    return bp.ravel()


def water_fill(v: np.ndarray, g: int, budget_bits: int, scale_bits: int = 16,
               max_width: int = 8):
    """Reverse water-filling under a per-token bit budget.

    Returns (widths [n_groups] int, theta).  theta is the breakpoint at which the scan
    stopped (inf when not even one group fits).  The widths it returns are b(theta)."""
    v = np.asarray(v, dtype=np.float64)
    theta = math.inf
    widths = widths_at(v, theta, max_width)
    for t in sorted(set(breakpoints(v, max_width).tolist()), reverse=True):
        # widths_at() evaluates log2 in floating point; exactly at a breakpoint that can
        # round either way, so the widths are counted from the breakpoints instead.
        w = _widths_by_count(v, t, max_width)
        if cost(w, g, scale_bits) > budget_bits:
            break
        theta, widths = t, w
    return widths, theta


def _widths_by_count(v: np.ndarray, theta: float, max_width: int) -> np.ndarray:
    """b_k(theta) as the number of group k's breakpoints that are >= theta; equal to
    widths_at() but free of log2 rounding exactly at a breakpoint."""
    j = np.arange(1, max_width + 1, dtype=np.float64)
    bp = v[:, None] * np.power(4.0, -(j - 0.5))[None, :]
    return np.sum(bp >= theta, axis=1).astype(np.int64)


def active_groups(widths: np.ndarray):
    """Indices of groups with a non-zero width (the others are dropped)."""
    return [k for k, b in enumerate(np.asarray(widths).tolist()) if b > 0]
