"""Rate-distortion quality harness: the codec's error against the bit budget, on the GPU path.

The pages disagree on whether the bit allocation matters.  The SPECTRA summary (Methodology,
second observation) states that allocating bits by channel energy clearly beats uniform
precision, especially below two bits; the ablation study (Core contributions 3, and its
practical advice) finds uniform allocation about as good as water-filling on synthetic data.
This harness measures both allocations on the same transform, budgets and synthetic regimes:

  regimes     Gaussian rows with eigenvalue decay i^-1.2; the same with every row Student-t(3)
              (heavy tails, the ablation study's Methodology); isotropic Gaussian rows;
  budgets     1.33, 2, 3 and 4 bits per original element, group scales included;
  allocation  "water" - the library's rounding reverse water-filling (spectra_calibrate);
              "uniform" - one width for the k leading groups (energy order) and nothing for the
              rest, k chosen by the same per-group variance model under the same budget;
              "water+e90", "water+gap2" - water-filling after the energy rank rule at 90 % or
              the spectral-gap rule at ratio 2 (spectra_rank_rule) has capped the rank;
              "water+robust" - water-filling on the outlier-robust calibration from the same
              rows (spatial-sign directions, median variances; spectra_calibrate robust);
              "water+vcorr" - water-filling with the least-squares value-latent correction
              folded into W_up_V (spectra_calibrate value_correction, same rows).

Per case the layer is calibrated on the host (G-weighted SVD), encoded and decoded by the GPU
kernels, and compared with exact float32 attention on the same inputs:
  relMSE_K, relMSE_V   sum |K^ - K|^2 / sum |K|^2 over the evaluation tokens (K^ = C^ W_up);
  relMSE_out, cos      error of the attention output over (sequence, query head);
  d2                   relMSE_out^2 + (1 - mean cos)^2: the point (relMSE, 1 - cos) of the
                       ablation study's two-dimensional error, as a squared distance (a reading:
                       the pages name the two components, not how they combine).

usage: python quality.py [--quick] [--json out.json]
"""
import argparse
import dataclasses
import json
import math
import sys
import time

import numpy as np

import spectral_transform_coding_amd as sp
from synth import configs as C
from synth import generators as gen

REGIMES = {
    "gauss_decay1.2": dict(decay=1.2, outlier_frac=0.0),
    "student_t3_decay1.2": dict(decay=1.2, outlier_frac=1.0),
    "isotropic": dict(decay=0.0, outlier_frac=0.0),
}
BUDGETS = (1.33, 2.0, 3.0, 4.0)


def log(msg):
    print(f"[quality {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def uniform_widths(sigma2, group_size, budget_bits, n_orig, scale_bits=16, max_width=8):
    """One width b for the k leading groups, zero after: the k (and b = the largest width the
    budget allows for k groups) minimising sum_kept v_g 4^-b + sum_dropped v_g, with v_g the
    mean latent variance of group g (energy order)."""
    v = np.asarray(sigma2, dtype=np.float64).reshape(-1, group_size).mean(axis=1)
    R = math.floor(budget_bits * n_orig)
    best = None
    for k in range(1, v.size + 1):
        b = min(max_width, (R - scale_bits * k) // (group_size * k))
        if b < 1:
            break
        dist = float((v[:k] * 4.0 ** (-b)).sum() + v[k:].sum())
        if best is None or dist < best[0]:
            best = (dist, k, b)
    _, k, b = best
    return np.array([b] * k + [0] * (v.size - k), dtype=np.uint8)


def run_case(wl, regime, budgets, batch, ctx, n_calib, device, rows_cache):
    import torch
    wl_r = dataclasses.replace(wl, **REGIMES[regime])
    d, dh, hq, nkv, g = wl.d_model, wl.d_head, wl.n_q_heads, wl.n_kv_heads, wl.group_size
    n_orig = nkv * dh
    q_basis = gen.basis_torch(wl_r, device)
    # calibration Gram matrix on the device in float64
    xc = gen.hidden_rows_torch(wl_r, n_calib, gen.STREAM_CALIB, q_basis, device).to(torch.bfloat16).double()
    G = (xc.T @ xc / n_calib).cpu().numpy()
    rows_host = xc.cpu().numpy()                        # the same rows, for the robust calibration
    del xc
    wk, wv, wq, _ = gen.projection_weights(wl_r)
    wk32 = torch.tensor(gen.to_bf16_f32(wk), device=device)
    wv32 = torch.tensor(gen.to_bf16_f32(wv), device=device)
    # evaluation rows and queries
    x = torch.stack([gen.hidden_rows_torch(wl_r, ctx, 100 + b, q_basis, device) for b in range(batch)])
    xb = x.to(torch.bfloat16)
    hq_rows = gen.hidden_rows_torch(wl_r, batch, gen.STREAM_QUERY, q_basis, device).to(torch.bfloat16).float()
    q = (hq_rows @ torch.tensor(gen.to_bf16_f32(wq), device=device)).view(batch, hq, dh).to(torch.bfloat16)
    xf = xb.float()
    K = xf @ wk32                                       # [B, T, n_kv dh] exact (fp32 products of bf16)
    V = xf @ wv32
    # exact attention per query head (GQA)
    scale = 1.0 / math.sqrt(dh)
    qf = q.float()
    o_ref = torch.empty((batch, hq, dh), device=device)
    for h in range(hq):
        kv = h * nkv // hq
        s = torch.einsum("btd,bd->bt", K[:, :, kv * dh:(kv + 1) * dh], qf[:, h]) * scale
        p = torch.softmax(s, dim=1)
        o_ref[:, h] = torch.einsum("bt,btd->bd", p, V[:, :, kv * dh:(kv + 1) * dh])
    # the full transform (every group active) for the uniform allocations
    full = sp.calibrate(G, wk, wv, nkv, dh, 1, wl.seg_rank, g, fixed_width=1)
    out = []
    for budget in budgets:
        cals = {
            "water": sp.calibrate(G, wk, wv, nkv, dh, 1, wl.seg_rank, g, budget_bits=budget),
            "water+e90": sp.calibrate(G, wk, wv, nkv, dh, 1, wl.seg_rank, g, budget_bits=budget,
                                      energy=0.90, rank_rule=sp.RANK_ENERGY),
            "water+gap2": sp.calibrate(G, wk, wv, nkv, dh, 1, wl.seg_rank, g, budget_bits=budget,
                                       gap_ratio=2.0, rank_rule=sp.RANK_GAP),
            "water+robust": sp.calibrate(None, wk, wv, nkv, dh, 1, wl.seg_rank, g, budget_bits=budget,
                                         rows=rows_host, robust=True),
            "water+vcorr": sp.calibrate(G, wk, wv, nkv, dh, 1, wl.seg_rank, g, budget_bits=budget,
                                        rows=rows_host, value_correction=True),
        }
        for alloc in ("water", "uniform", "water+e90", "water+gap2", "water+robust", "water+vcorr"):
            if alloc != "uniform":
                cal = cals[alloc]
                wk_w, wv_w = cal["widths_k"].reshape(-1), cal["widths_v"].reshape(-1)
                tk, tv = cal["w_down_t_k"], cal["w_down_t_v"]
                uk, uv = cal["w_up_k"], cal["w_up_v"]
            else:
                wk_w = uniform_widths(full["sigma2_k"], g, budget, n_orig)
                wv_w = uniform_widths(full["sigma2_v"], g, budget, n_orig)
                mk = np.repeat(wk_w > 0, g)
                mv = np.repeat(wv_w > 0, g)
                tk, tv = full["w_down_t_k"][mk], full["w_down_t_v"][mv]
                uk, uv = full["w_up_k"][mk], full["w_up_v"][mv]
            lay = sp.Layout(d, hq, nkv, dh, 1, wl.seg_rank, g, wk_w, wv_w)
            wdt = torch.tensor(gen.to_bf16_f32(np.concatenate([tk, tv], axis=0)), device=device).to(torch.bfloat16)
            ck = torch.zeros(lay.cache_bytes(sp.TENSOR_K, batch, ctx), dtype=torch.uint8, device=device)
            cv = torch.zeros(lay.cache_bytes(sp.TENSOR_V, batch, ctx), dtype=torch.uint8, device=device)
            sp.encode_append(lay, xb, wdt, ck, cv, ctx, [0] * batch)
            chat_k = sp.unpack_dequant(lay, sp.TENSOR_K, ck, ctx, batch, 0, ctx)
            chat_v = sp.unpack_dequant(lay, sp.TENSOR_V, cv, ctx, batch, 0, ctx)
            upk = torch.tensor(gen.to_bf16_f32(uk), device=device)
            upv = torch.tensor(gen.to_bf16_f32(uv), device=device)
            rel_k = float(((chat_k @ upk - K) ** 2).sum() / (K ** 2).sum())
            rel_v = float(((chat_v @ upv - V) ** 2).sum() / (V ** 2).sum())
            o = sp.decode_attn(lay, q, ck, cv, ctx, [ctx] * batch, upk.to(torch.bfloat16),
                               upv.to(torch.bfloat16), scale)
            torch.cuda.synchronize()
            rel_o = float(((o - o_ref) ** 2).sum() / (o_ref ** 2).sum())
            cos = float(torch.nn.functional.cosine_similarity(o.reshape(-1, dh), o_ref.reshape(-1, dh), dim=1).mean())
            bits = sum(g * int(b) + 16 for b in wk_w if b) / n_orig     # codes plus one fp16 scale per group
            row = dict(regime=regime, budget=budget, alloc=alloc, bits_per_elem_k=round(bits, 3),
                       r_act_k=int(lay.r_act(sp.TENSOR_K)), r_act_v=int(lay.r_act(sp.TENSOR_V)),
                       widths_k=[int(b) for b in wk_w], relmse_k=rel_k, relmse_v=rel_v,
                       relmse_out=rel_o, cos=cos, d2=rel_o ** 2 + (1.0 - cos) ** 2)
            log(f"{regime:22s} b={budget:4.2f} {alloc:12s} r_act {row['r_act_k']:3d}  relMSE_K {rel_k:.4f}  "
                f"relMSE_V {rel_v:.4f}  out {rel_o:.5f}  cos {cos:.5f}")
            out.append(row)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--quick", action="store_true", help="one regime, two budgets, short context")
    ap.add_argument("--json", default=None, help="write the rows here")
    args = ap.parse_args()
    import torch
    if not torch.cuda.is_available():
        sys.exit("quality.py needs a GPU (it runs the library's kernels)")
    device = torch.device("cuda:0")
    wl = C.LLAMA8B_4BIT
    regimes = ["gauss_decay1.2"] if args.quick else list(REGIMES)
    budgets = (2.0, 4.0) if args.quick else BUDGETS
    batch, ctx, n_calib = (2, 1024, 8192) if args.quick else (4, 4096, 32768)
    rows = []
    for regime in regimes:
        log(f"regime {regime}: calibrating on {n_calib} rows, evaluating {batch} x {ctx} tokens")
        rows += run_case(wl, regime, budgets, batch, ctx, n_calib, device, None)
    hdr = f"{'regime':22s} {'bits':>5s} {'alloc':12s} {'r_act':>5s} {'relMSE_K':>9s} {'relMSE_V':>9s} {'relMSE_out':>10s} {'1-cos':>9s} {'d2':>9s}"
    print(hdr)
    for r in rows:
        print(f"{r['regime']:22s} {r['budget']:5.2f} {r['alloc']:12s} {r['r_act_k']:5d} {r['relmse_k']:9.5f} "
              f"{r['relmse_v']:9.5f} {r['relmse_out']:10.6f} {1 - r['cos']:9.2e} {r['d2']:9.2e}")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(dict(workload=wl.name, batch=batch, ctx=ctx, calib_rows=n_calib, rows=rows), f, indent=1)


if __name__ == "__main__":
    main()
