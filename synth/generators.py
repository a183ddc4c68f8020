"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module draws random numbers and shapes their distribution; it computes no step of the
codec (no projection onto a latent, no bit allocation, no quantization, no packing, no
attention).  Both the CPU oracle and the HIP path receive what it returns as plain inputs.

Hidden states follow the synthetic-regime idea of the KV-cache ablation study
("Ablation, Statistical Inference, and Validation for KV-Cache Compression", methodology
section): Gaussian rows with a controlled eigenvalue decay under a random orthogonal basis,
plus a small fraction of heavy-tailed Student-t(3) rows.

Seeds: NumPy PCG64 with seed = 1000 * workload_index + stream, streams:
  0 basis, 1 calibration rows, 2 W_K, 3 W_V, 4 W_Q, 5 W_O,
  100 + b rows of sequence b, 10**6 + step streaming rows, 7 queries, 8 latent rows.
"""
import math
import numpy as np

from .configs import ALL, Workload

STREAM_BASIS, STREAM_CALIB, STREAM_WK, STREAM_WV, STREAM_WQ, STREAM_WO = 0, 1, 2, 3, 4, 5
STREAM_QUERY, STREAM_LATENT = 7, 8


def workload_index(wl: Workload) -> int:
    for i, w in enumerate(ALL):
        if w.name == wl.name:
            return i + 1
    return 99


def rng_for(wl: Workload, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * workload_index(wl) + stream))


def cov_spectrum(d: int, decay: float) -> np.ndarray:
    """Eigenvalues lambda_i = c * i^-decay (i = 1..d) normalised so that they sum to d."""
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-decay)
    return lam * (d / lam.sum())


def haar_orthogonal(d: int, rng: np.random.Generator) -> np.ndarray:
    """Random orthogonal matrix: QR of a Gaussian matrix with the sign of R's diagonal fixed."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def basis(wl: Workload) -> np.ndarray:
    return haar_orthogonal(wl.d_model, rng_for(wl, STREAM_BASIS))


def _outlier_factors(n: int, frac: float, rng: np.random.Generator) -> np.ndarray:
    """Per-row factor sqrt(3 / chi2_3) on a fraction `frac` of rows (a multivariate t(3) row
    is a Gaussian row times this factor); 1 elsewhere."""
    f = np.ones(n)
    if frac > 0:
        pick = rng.random(n) < frac
        chi = rng.chisquare(3.0, size=int(pick.sum()))
        f[pick] = np.sqrt(3.0 / chi)
    return f


def hidden_rows(wl: Workload, n: int, stream: int, q_basis: np.ndarray = None) -> np.ndarray:
    """n rows h = z diag(sqrt(lambda)) Q^T (float64), with the workload's outlier rows."""
    rng = rng_for(wl, stream)
    lam = cov_spectrum(wl.d_model, wl.decay)
    z = rng.standard_normal((n, wl.d_model)) * np.sqrt(lam)[None, :]
    z *= _outlier_factors(n, wl.outlier_frac, rng)[:, None]
    if q_basis is None:
        q_basis = basis(wl)
    return z @ q_basis.T


def projection_weights(wl: Workload):
    """W_K, W_V, W_Q ~ N(0, 1/d_model); W_O ~ N(0, 1/(Hq d_h)).  float64."""
    d, kv = wl.d_model, wl.n_kv_heads * wl.d_head
    qd = wl.n_q_heads * wl.d_head
    wk = rng_for(wl, STREAM_WK).standard_normal((d, kv)) / math.sqrt(d)
    wv = rng_for(wl, STREAM_WV).standard_normal((d, kv)) / math.sqrt(d)
    wq = rng_for(wl, STREAM_WQ).standard_normal((d, qd)) / math.sqrt(d)
    wo = rng_for(wl, STREAM_WO).standard_normal((qd, d)) / math.sqrt(qd)
    return wk, wv, wq, wo


def latent_rows(sigma2: np.ndarray, n: int, rng: np.random.Generator,
                outlier_frac: float = 0.0) -> np.ndarray:
    """n rows with independent coordinates of variances sigma2 (float64), with outlier rows.
    Used to build large caches without forming d_model-wide rows."""
    c = rng.standard_normal((n, sigma2.size)) * np.sqrt(np.asarray(sigma2))[None, :]
    c *= _outlier_factors(n, outlier_frac, rng)[:, None]
    return c


def gaussian(shape, rng: np.random.Generator, scale: float = 1.0) -> np.ndarray:
    return rng.standard_normal(shape) * scale


def to_bf16_f32(a: np.ndarray) -> np.ndarray:
    """Round float values to bfloat16 (nearest, ties to even) and return them as float32."""
    x = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = ((x >> 16) & 1) + 0x7FFF
    y = ((x + rounding) >> 16) << 16
    out = y.astype(np.uint32).view(np.float32)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of to_bf16_f32(a)."""
    return (to_bf16_f32(a).view(np.uint32) >> 16).astype(np.uint16)


def input_dtype_round(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values as the GPU will see them: float32, or bfloat16 widened to float32."""
    return to_bf16_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


# ------------------------------------------------------------------ device-side variants
# Same recipes drawn with torch's generator on the GPU, for workloads whose rows are too many to
# draw on the host (hundreds of thousands of d_model-wide rows).  They yield different numbers
# from the NumPy recipes above (a different generator), with the same distribution.

def torch_generator(wl: Workload, stream: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(1000 * workload_index(wl) + stream)
    return g


def hidden_rows_torch(wl: Workload, n: int, stream: int, q_basis, device, dtype=None):
    """n rows h = z diag(sqrt(lambda)) Q^T on the device (float32), with outlier rows."""
    import torch
    g = torch_generator(wl, stream, device)
    lam = torch.tensor(cov_spectrum(wl.d_model, wl.decay), dtype=torch.float32, device=device)
    z = torch.randn((n, wl.d_model), generator=g, device=device, dtype=torch.float32) * lam.sqrt()
    if wl.outlier_frac > 0:
        pick = torch.rand(n, generator=g, device=device) < wl.outlier_frac
        chi = (torch.randn((n, 3), generator=g, device=device) ** 2).sum(dim=1)
        f = torch.where(pick, torch.sqrt(3.0 / chi), torch.ones_like(chi))
        z = z * f[:, None]
    return z @ q_basis.T


def basis_torch(wl: Workload, device):
    """Haar orthogonal basis drawn on the device (float32)."""
    import torch
    g = torch_generator(wl, STREAM_BASIS, device)
    a = torch.randn((wl.d_model, wl.d_model), generator=g, device=device, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    return (q * torch.sign(torch.diagonal(r))[None, :]).to(torch.float32)
