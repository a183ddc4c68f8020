"""Per-token group quantiser (oracle).

[SPECTRA] SPECTRA pipeline, stage 3: at inference each token is down-projected, quantised
per token and appended to the latent cache; stage 2: adjacent coordinates form a group
with one width.  The tiny workload fixes fp16 per-token group scales.

Reading (the pages give no quantiser formula): a symmetric uniform quantiser whose 2^b cells
tile [-A, A], A = max_j |c_j| over the group's coordinates for this token, reconstructing at
cell midpoints:
    s  = fp16_rne(A * 2^(1-b))            (fp16 overflow saturates to 65504)
    u_j = clamp(rint_half_even(c_j / s + (2^b - 1)/2), 0, 2^b - 1)   (u = 0 when s = 0)
    c^_j = s * (u_j - (2^b - 1)/2)
The code is computed in float32 exactly as written (a correctly rounded float32 division,
then a float32 addition, then round-half-even), so that any implementation given the same
float32 latent produces the same codes.  The dequantised value is exact in float32: an
11-bit fp16 significand times a half-integer of at most 8 bits needs at most 19 bits.
"""
import numpy as np

FP16_MAX = np.float32(65504.0)


def scales_fp16(c32: np.ndarray, b: int) -> np.ndarray:
    """fp16 scale per row of c32 [..., g] (returned as float16)."""
    c32 = np.asarray(c32, dtype=np.float32)
    A = np.max(np.abs(c32), axis=-1)
    s32 = (A * np.float32(2.0 ** (1 - b))).astype(np.float32)    # exact power-of-two scaling
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)                              # round to nearest even
    s16 = np.where(np.isinf(s16), np.float16(FP16_MAX), s16)
    return s16


def codes(c32: np.ndarray, s16: np.ndarray, b: int) -> np.ndarray:
    """uint8 codes for c32 [..., g] with scales s16 [...]."""
    c32 = np.asarray(c32, dtype=np.float32)
    s = np.asarray(s16, dtype=np.float16).astype(np.float32)[..., None]
    h = np.float32((2 ** b - 1) / 2.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.divide(c32, s, dtype=np.float32)
        x = np.add(x, h, dtype=np.float32)
    u = np.rint(x)
    u = np.where(s == 0, 0.0, u)
    u = np.clip(u, 0, 2 ** b - 1)
    return u.astype(np.uint8)


def quantize(c32: np.ndarray, b: int):
    """(codes uint8 [..., g], scales float16 [...]) for one group width b >= 1."""
    s16 = scales_fp16(c32, b)
    return codes(c32, s16, b), s16


def dequantize(u: np.ndarray, s16: np.ndarray, b: int) -> np.ndarray:
    """c^ = s * (u - (2^b-1)/2) as float64 (exactly the float32 value)."""
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)[..., None]
    return s * (np.asarray(u, dtype=np.float64) - (2 ** b - 1) / 2.0)


def quantize_latent(c32: np.ndarray, widths_active, g: int):
    """Quantise latent rows c32 [n, r_act] whose columns are the active groups in order,
    with widths_active[i] the width of the i-th active group.
    Returns (codes uint8 [n, r_act], scales float16 [n, n_active])."""
    c32 = np.asarray(c32, dtype=np.float32)
    n = c32.shape[0]
    na = len(widths_active)
    assert c32.shape[1] == na * g
    u = np.zeros((n, na * g), dtype=np.uint8)
    s = np.zeros((n, na), dtype=np.float16)
    for i, b in enumerate(widths_active):
        cu, cs = quantize(c32[:, i * g:(i + 1) * g], int(b))
        u[:, i * g:(i + 1) * g] = cu
        s[:, i] = cs
    return u, s


def dequantize_latent(u: np.ndarray, s16: np.ndarray, widths_active, g: int) -> np.ndarray:
    n = u.shape[0]
    out = np.zeros((n, len(widths_active) * g), dtype=np.float64)
    for i, b in enumerate(widths_active):
        out[:, i * g:(i + 1) * g] = dequantize(u[:, i * g:(i + 1) * g], s16[:, i], int(b))
    return out
