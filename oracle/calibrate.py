"""Offline calibration: transform + widths for one layer (oracle, float64).

[SPECTRA] SPECTRA pipeline stages 1-2 and 3 (system integration: W_down, W_up and the W_O fix
are folded into the weights).  Per tensor (K, V) and per segment (one segment spanning every
key/value head, or one segment per head as in [SPECTRAL-KV] Technical principle, 1):
  M = W_s^T G W_s  ->  eigenvectors V (descending eigenvalues)  ->  V_r, sigma^2 = lambda_1..r
  widths = water-filling over group variances of sigma^2 (or one fixed width)
  active groups (width > 0) -> W_down_s = W_s V_r[:, active],  W_up_s = V_r[:, active]^T
The per-tensor bit budget is R = floor(budget_bits * n_kv * d_head / n_seg) per token and
segment, scales included.
"""
import math
import numpy as np

from . import transform, allocation


def calibrate_tensor(G, W, n_seg, seg_rank, g, budget_bits, fixed_width=None, energy=None,
                     scale_bits=16, max_width=8):
    d, n = W.shape
    seg_cols = n // n_seg
    R = int(math.floor(budget_bits * seg_cols + 1e-9))
    downs, ups, widths, sig, thetas, erank = [], [], [], [], [], []
    for s in range(n_seg):
        Ws = W[:, s * seg_cols:(s + 1) * seg_cols]
        lam, V = transform.g_weighted_eig(G, Ws)
        erank.append(transform.energy_rank(lam, energy) if energy else -1)
        Vr = V[:, :seg_rank]
        s2 = lam[:seg_rank]
        v = allocation.group_variances(s2, g)
        if fixed_width is not None:
            w = np.full(v.size, fixed_width, dtype=np.int64)
            th = math.nan
        else:
            w, th = allocation.water_fill(v, g, R, scale_bits, max_width)
        act = allocation.active_groups(w)
        cols = np.concatenate([np.arange(k * g, (k + 1) * g) for k in act]) if act else np.zeros(0, int)
        downs.append(Ws @ Vr[:, cols])
        ups.append(Vr[:, cols].T)
        widths.append(w)
        sig.append(s2)
        thetas.append(th)
    return dict(w_down=np.concatenate(downs, axis=1), w_up=np.concatenate(ups, axis=0),
                widths=np.stack(widths), sigma2=np.stack(sig), theta=np.array(thetas),
                energy_rank=np.array(erank), budget=R)


def calibrate(G, W_K, W_V, n_seg, seg_rank, g, budget_bits, fixed_width=None, energy=None,
              scale_bits=16, max_width=8):
    k = calibrate_tensor(G, W_K, n_seg, seg_rank, g, budget_bits, fixed_width, energy, scale_bits, max_width)
    v = calibrate_tensor(G, W_V, n_seg, seg_rank, g, budget_bits, fixed_width, energy, scale_bits, max_width)
    return dict(k=k, v=v, w_down=np.concatenate([k["w_down"], v["w_down"]], axis=1))
