"""Shared test utilities: layouts, synthetic caches packed by the oracle, device transfer."""
import math

import numpy as np

from oracle import layout as OL, attention as OA, quant as OQ
from synth import generators as gen
import spectral_transform_coding_amd as sp


def make_layouts(d_model, n_q, n_kv, d_head, n_seg, seg_rank, g, widths_k, widths_v):
    """(oracle layout, library layout) with the same shape."""
    wk = np.asarray(widths_k, dtype=np.int64).reshape(n_seg, -1)
    wv = np.asarray(widths_v, dtype=np.int64).reshape(n_seg, -1)
    return (OL.Layout(d_model, n_q, n_kv, d_head, n_seg, seg_rank, g, wk, wv),
            sp.Layout(d_model, n_q, n_kv, d_head, n_seg, seg_rank, g, wk, wv))


def orthonormal_rows(r, n, rng):
    """[r x n] with orthonormal rows (a W_up stand-in)."""
    q, _ = np.linalg.qr(rng.standard_normal((n, r)))
    return q.T.copy()


def build_caches(olay, batch, cap, ctx, rng, sigma_decay=1.0, outlier_frac=0.0, scale=1.0):
    """Caches [batch, nblk, block_bytes] (K and V) holding ctx[b] tokens per sequence, packed
    by the oracle from synthetic latent rows with decaying variances."""
    ck = olay.empty_cache("K", batch, cap)
    cv = olay.empty_cache("V", batch, cap)
    lat = {}
    for kind, cache in (("K", ck), ("V", cv)):
        r = olay.r_act(kind)
        s2 = scale * np.arange(1, r + 1, dtype=np.float64) ** (-sigma_decay) * 4.0
        for b in range(batch):
            n = int(ctx[b])
            c = gen.latent_rows(s2, n, rng, outlier_frac).astype(np.float32)
            u, s = OQ.quantize_latent(c, olay.widths_active(kind), olay.g)
            OL.write_tokens(olay, kind, cache, b, np.arange(n), u, s)
            lat[(kind, b)] = c
    return ck, cv, lat


def max_rel_err(out, ref):
    """max over rows of ||out - ref||_inf / ||ref||_inf (rows = last axis vectors)."""
    out = np.asarray(out, np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    worst = 0.0
    for o, r in zip(out, ref):
        den = np.abs(r).max()
        if den == 0:
            if np.abs(o).max() != 0:
                return math.inf
            continue
        worst = max(worst, np.abs(o - r).max() / den)
    return worst


def to_dev(a, dtype, device="cuda"):
    """numpy float -> torch tensor on the device in 'f32' or 'bf16' (nearest-even rounding)."""
    import torch
    if dtype == "bf16":
        bits = gen.f32_to_bf16_bits(np.asarray(a, np.float32))
        return torch.from_numpy(bits.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_bytes(cache, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(cache).reshape(-1)).to(device)
