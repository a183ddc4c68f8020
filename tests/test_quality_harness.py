"""The rate-distortion harness (quality.py): its uniform allocation on the host, and on the GPU its
error measurement checked against the oracle and a short run's sanity.

The harness compares the library's water-filled widths with one uniform width over the k leading
groups under the same budget (the ablation study's uniform-allocation variant; "Ablation,
Statistical Inference, and Validation for KV-Cache Compression", practical advice).
"""
import math
import sys

import numpy as np
import pytest

import quality as Q
from oracle import quant as OQ
from synth import generators as gen


def _cost(widths, g, scale_bits=16):
    return sum(g * int(b) + scale_bits for b in widths if b)


@pytest.mark.parametrize("budget", [1.0, 1.33, 2.0, 3.0, 4.0, 6.0])
def test_uniform_widths_fit_the_budget_and_minimise_the_model(budget):
    rng = np.random.default_rng(3)
    g, groups, n_orig = 16, 32, 1024
    sigma2 = np.sort(rng.gamma(0.5, 1.0, groups * g))[::-1] * np.repeat(np.arange(1, groups + 1) ** -1.5, g)
    w = Q.uniform_widths(sigma2, g, budget, n_orig)
    R = math.floor(budget * n_orig)
    assert _cost(w, g) <= R
    kept = w[w > 0]
    assert kept.size >= 1 and np.all(kept == kept[0])                 # one width
    assert np.all(w[:kept.size] > 0) and np.all(w[kept.size:] == 0)     # leading groups
    # brute force over every (k, b) that fits: none has a smaller model distortion
    v = sigma2.reshape(groups, g).mean(axis=1)
    model = lambda k, b: float((v[:k] * 4.0 ** (-b)).sum() + v[k:].sum())
    got = model(kept.size, int(kept[0]))
    for k in range(1, groups + 1):
        for b in range(1, 9):
            if _cost([b] * k, g) <= R:
                assert got <= model(k, b) + 1e-12


@pytest.mark.gpu
def test_harness_reconstruction_error_matches_the_oracle():
    """relMSE_K as the harness forms it (GPU codes unpacked, lifted by W_up) equals the oracle's
    quantisation of the same float32 latents, dequantised and lifted in float64."""
    import torch
    import spectral_transform_coding_amd as sp
    print("[quality] reconstruction error vs oracle", flush=True)
    dev = torch.device("cuda:0")
    d, hq, nkv, dh, r, g = 512, 4, 2, 64, 64, 16
    rng = np.random.default_rng(5)
    wk = rng.standard_normal((d, nkv * dh)) / math.sqrt(d)
    wv = rng.standard_normal((d, nkv * dh)) / math.sqrt(d)
    lam = gen.cov_spectrum(d, 1.2)
    xc = rng.standard_normal((4096, d)) * np.sqrt(lam)
    G = xc.T @ xc / xc.shape[0]
    cal = sp.calibrate(G, wk, wv, nkv, dh, 1, r, g, budget_bits=2.0)
    lay = sp.Layout(d, hq, nkv, dh, 1, r, g, cal["widths_k"].reshape(-1), cal["widths_v"].reshape(-1))
    T = 300
    x = gen.to_bf16_f32(rng.standard_normal((1, T, d)) * np.sqrt(lam))
    wdt = gen.to_bf16_f32(np.concatenate([cal["w_down_t_k"], cal["w_down_t_v"]], axis=0))
    xd = torch.tensor(x, device=dev).to(torch.bfloat16)
    wd = torch.tensor(wdt, device=dev).to(torch.bfloat16)
    ck = torch.zeros(lay.cache_bytes(sp.TENSOR_K, 1, T), dtype=torch.uint8, device=dev)
    cv = torch.zeros(lay.cache_bytes(sp.TENSOR_V, 1, T), dtype=torch.uint8, device=dev)
    rk, rv = lay.r_act(sp.TENSOR_K), lay.r_act(sp.TENSOR_V)
    lat = torch.zeros((T, rk + rv), dtype=torch.float32, device=dev)
    sp.encode_append(lay, xd, wd, ck, cv, T, [0], latent_out=lat)
    chat = sp.unpack_dequant(lay, sp.TENSOR_K, ck, T, 1, 0, T)[0]
    upk = gen.to_bf16_f32(cal["w_up_k"])
    K = x[0].astype(np.float64) @ gen.to_bf16_f32(wk).astype(np.float64)
    gpu = (chat.double() @ torch.tensor(upk, dtype=torch.float64, device=dev)).cpu().numpy()
    widths = [int(b) for b in cal["widths_k"].reshape(-1) if b]
    u, s16 = OQ.quantize_latent(lat[:, :rk].cpu().numpy(), widths, g)
    ref = OQ.dequantize_latent(u, s16, widths, g) @ upk.astype(np.float64)
    rel_gpu = ((gpu - K) ** 2).sum() / (K ** 2).sum()
    rel_ref = ((ref - K) ** 2).sum() / (K ** 2).sum()
    print(f"    relMSE_K gpu {rel_gpu:.6e} oracle {rel_ref:.6e}", flush=True)
    assert abs(rel_gpu - rel_ref) <= 1e-9 * max(rel_ref, 1e-30) + 1e-12
    assert 0.0 < rel_ref < 1.0


@pytest.mark.gpu
def test_harness_quick_run_is_sane():
    """A short run: more bits never raise the reconstruction or output error by much, and the
    output stays close to exact attention."""
    import torch
    print("[quality] quick run", flush=True)
    rows = Q.run_case(Q.C.LLAMA8B_4BIT, "gauss_decay1.2", (2.0, 4.0), 1, 512, 4096,
                      torch.device("cuda:0"), None)
    by = {(r["alloc"], r["budget"]): r for r in rows}
    for alloc in ("water", "uniform", "water+robust", "water+vcorr"):
        lo, hi = by[(alloc, 2.0)], by[(alloc, 4.0)]
        assert hi["relmse_k"] < lo["relmse_k"] and hi["relmse_v"] < lo["relmse_v"]
        assert hi["cos"] > 0.9
        assert hi["bits_per_elem_k"] <= 4.0 and lo["bits_per_elem_k"] <= 2.0
