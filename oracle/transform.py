"""Activation-weighted spectral transform (oracle, float64).

[SPECTRA] Methodology, third observation: a channel's importance depends on how the input
activations drive it, so the transform is weighted by the activation Gram matrix
G = E[h^T h].  [SPECTRA] SPECTRA pipeline, stage 1: W_K and W_V are factorised by an SVD
weighted by G (whitening the weights with G^(1/2)); the result is an energy-ordered latent C
whose coordinates are orthogonal (second-moment orthogonal, Core contributions) and sorted
by variance.

Reading used here: the right singular vectors of G^(1/2) W are the eigenvectors V of
M = W^T G W, with squared singular values = eigenvalues.  The down-projection is W V_r, the
up-projection V_r^T, so a token's latent is c = h W V_r = k V_r, where k = h W is its key;
this is the projection k_latent = k V_r of [SPECTRAL-KV] Technical principle, 2.
No inverse of G is formed, so a singular G is fine.
"""
import numpy as np
from scipy import stats as _stats


def gram(rows: np.ndarray) -> np.ndarray:
    """G = E[h^T h] over calibration rows (uncentred second moment), float64."""
    h = np.asarray(rows, dtype=np.float64)
    return h.T @ h / h.shape[0]


def canonical_signs(vecs: np.ndarray) -> np.ndarray:
    """Flip each column so that its entry of largest magnitude is positive (first such index
    on ties).  Any sign is a valid eigenvector; this only fixes one."""
    v = np.array(vecs, dtype=np.float64, copy=True)
    idx = np.argmax(np.abs(v), axis=0)          # argmax returns the first maximum
    sgn = np.sign(v[idx, np.arange(v.shape[1])])
    sgn[sgn == 0] = 1.0
    return v * sgn[None, :]


def g_weighted_eig(G: np.ndarray, W: np.ndarray):
    """Eigen-decomposition of M = W^T G W, eigenvalues descending (ties keep index order),
    canonical signs.  Returns (lam [n], V [n x n])."""
    G = np.asarray(G, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    M = W.T @ G @ W
    M = 0.5 * (M + M.T)
    lam, V = np.linalg.eigh(M)                  # ascending
    order = np.argsort(-lam, kind="stable")
    lam = lam[order]
    V = V[:, order]
    return lam, canonical_signs(V)


def energy_rank(lam: np.ndarray, tau: float) -> int:
    """Smallest r with sum_{i<=r} lam_i / sum_i lam_i >= tau ([SPECTRAL-KV] Technical
    principle, 1: effective rank at a target energy such as 95 %).  Negative round-off
    eigenvalues count as zero."""
    lam = np.clip(np.asarray(lam, dtype=np.float64), 0.0, None)
    tot = lam.sum()
    if tot <= 0:
        return 1
    frac = np.cumsum(lam) / tot
    return int(np.searchsorted(frac, tau - 1e-15) + 1)


def gap_rank(lam: np.ndarray, r_max: int, ratio: float) -> int:
    """Rank trimmed at a spectral gap: among the leading r_max eigenvalues, the index i
    (1 <= i < r_max) of the largest ratio lam_i / lam_{i+1} (the first on ties); the rank is
    cut to i when that ratio reaches `ratio`, else r_max is kept.  Eigenvalues at or below zero
    count as 1e-300.  A reading of the ablation study's spectral-gap criterion for trimming the
    estimated dimension ("Ablation, Statistical Inference, and Validation for KV-Cache
    Compression", Core contributions 3); the pages name the criterion, not its form."""
    lam = np.maximum(np.asarray(lam[:r_max], dtype=np.float64), 1e-300)
    if lam.size < 2:
        return int(r_max)
    q = lam[:-1] / lam[1:]
    i = int(np.argmax(q))
    return i + 1 if q[i] >= ratio else int(r_max)


# Median of a chi-squared variable with one degree of freedom, (Phi^-1(3/4))^2: the median of
# (y . u)^2 for Gaussian rows is this times the variance along u.
CHI2_1_MEDIAN = float(_stats.norm.ppf(0.75) ** 2)


def robust_eig(Y: np.ndarray):
    """Outlier-robust eigen-decomposition of the second moment of projected rows Y [n x m]
    (y = h W_s), for heavy-tailed calibration rows.  The ablation study ("Ablation, Statistical
    Inference, and Validation for KV-Cache Compression", performance in specific regimes) finds
    the sample covariance corrupted by outliers on Student-t data, shifting the calibrated
    basis; it names no remedy.  Reading used here, for rows that are a common shape scaled by a
    random factor per row:
      directions  eigenvectors of the spatial-sign second moment S = mean of y y^T / |y|^2 over
                  the rows with y != 0 (each row's scale drops out);
      variances   along each direction u, the median over all rows of (y . u)^2 divided by
                  CHI2_1_MEDIAN (Gaussian rows give their variance; a per-row scale mixture
                  multiplies every direction's value by one common factor, which leaves the
                  water-filled widths and the rank rules unchanged).
    Returns (lam [m], V [m x m]): lam descending (ties keep the order of S's eigenvalues,
    descending), canonical signs."""
    Y = np.asarray(Y, dtype=np.float64)
    n, m = Y.shape
    nrm2 = (Y * Y).sum(axis=1)
    nz = nrm2 > 0
    S = np.zeros((m, m))
    if nz.any():
        Yn = Y[nz] / np.sqrt(nrm2[nz])[:, None]
        S = Yn.T @ Yn / int(nz.sum())
    S = 0.5 * (S + S.T)
    mu, U = np.linalg.eigh(S)
    U = U[:, np.argsort(-mu, kind="stable")]
    lam = np.median((Y @ U) ** 2, axis=0) / CHI2_1_MEDIAN
    order = np.argsort(-lam, kind="stable")
    return lam[order], canonical_signs(U[:, order])
