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

from . import transform, allocation, quant


def calibrate_tensor(G, W, n_seg, seg_rank, g, budget_bits, fixed_width=None, energy=None,
                     scale_bits=16, max_width=8, rank_rule="fixed", gap_ratio=None, rows=None, robust=False):
    """rank_rule limits the leading groups that receive bits: "fixed" (seg_rank), "energy" (the
    energy rank at `energy`, [SPECTRAL-KV] Technical principle 1) or "gap" (transform.gap_rank
    with `gap_ratio`); the kept rank is rounded up to whole groups, later groups get width 0.
    With robust=True, each segment's eigen-pairs come from transform.robust_eig of the
    projected calibration rows (rows [n x d]) W_s instead of from M = W_s^T G W_s (G is then
    unused)."""
    d, n = W.shape
    seg_cols = n // n_seg
    R = int(math.floor(budget_bits * seg_cols + 1e-9))
    downs, ups, widths, sig, thetas, erank = [], [], [], [], [], []
    for s in range(n_seg):
        Ws = W[:, s * seg_cols:(s + 1) * seg_cols]
        if robust:
            lam, V = transform.robust_eig(np.asarray(rows, dtype=np.float64) @ Ws)
        else:
            lam, V = transform.g_weighted_eig(G, Ws)
        er = transform.energy_rank(lam, energy) if energy else -1
        erank.append(er)
        Vr = V[:, :seg_rank]
        s2 = lam[:seg_rank]
        v = allocation.group_variances(s2, g)
        cap = seg_rank
        if rank_rule == "energy":
            cap = min(cap, er)
        elif rank_rule == "gap":
            cap = transform.gap_rank(lam, seg_rank, gap_ratio)
        else:
            assert rank_rule == "fixed", rank_rule
        cg = -(-cap // g)
        if fixed_width is not None:
            w = np.array([fixed_width] * cg + [0] * (v.size - cg), dtype=np.int64)
            th = math.nan
        else:
            wc, th = allocation.water_fill(v[:cg], g, R, scale_bits, max_width)
            w = np.concatenate([np.asarray(wc, dtype=np.int64), np.zeros(v.size - cg, dtype=np.int64)])
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


def value_correction(rows, w_down_s, widths_s, g):
    """Least-squares correction of a segment's value latents for quantisation.  [SPECTRA]
    SPECTRA pipeline stage 1 folds a closed-form correction of W_O into the weights; the pages
    give no formula.  Reading: over the calibration rows, the exact latents C = rows W_down_s
    (float64) and their dequantised values C^ (C rounded to float32, quantised and dequantised
    by quant with the segment's active widths) give F = argmin |C - C^ F|^2 = (C^T C^)^-1 C^T C;
    the up-projection becomes F W_up_s, so a cached value is rebuilt as c^ F W_up.  Returns F
    [r_act_s x r_act_s]."""
    C = np.asarray(rows, dtype=np.float64) @ np.asarray(w_down_s, dtype=np.float64)
    act = [int(b) for b in widths_s if b > 0]
    u, s16 = quant.quantize_latent(C.astype(np.float32), act, g)
    Ch = quant.dequantize_latent(u, s16, act, g)
    return np.linalg.solve(Ch.T @ Ch, Ch.T @ C)


def calibrate(G, W_K, W_V, n_seg, seg_rank, g, budget_bits, fixed_width=None, energy=None,
              scale_bits=16, max_width=8, rank_rule="fixed", gap_ratio=None, rows=None, robust=False,
              vcorr=False):
    """Both tensors; with vcorr=True, W_up_V of each segment is replaced by
    value_correction(...) W_up_V (calibration rows `rows` required)."""
    k = calibrate_tensor(G, W_K, n_seg, seg_rank, g, budget_bits, fixed_width, energy, scale_bits, max_width,
                         rank_rule, gap_ratio, rows, robust)
    v = calibrate_tensor(G, W_V, n_seg, seg_rank, g, budget_bits, fixed_width, energy, scale_bits, max_width,
                         rank_rule, gap_ratio, rows, robust)
    if vcorr:
        col = 0
        ups = []
        for s in range(n_seg):
            ns = int(sum(g for b in v["widths"][s] if b > 0))
            F = value_correction(rows, v["w_down"][:, col:col + ns], v["widths"][s], g)
            ups.append(F @ v["w_up"][col:col + ns])
            col += ns
        v["w_up"] = np.concatenate(ups, axis=0) if ups else v["w_up"]
    return dict(k=k, v=v, w_down=np.concatenate([k["w_down"], v["w_down"]], axis=1))
