"""GPU parity on the benchmark's own headline inputs: the Llama-shaped layer (4 bits per element,
batch 16 x 32 768) built exactly as bench.py builds it.  Rows are drawn on the GPU with 1 %
Student-t(3) rows, G is their Gram matrix, spectra_calibrate gives the transform and widths,
the GPU encoder fills the caches and the queries come from the same generator.

Heavy-tailed tokens carry large scales on every latent coordinate, so the rounding of the
matrix-core operands reaches into every group's share of the score ("Ablation, Statistical
Inference, and Validation for KV-Cache Compression", Core contributions 3, on heavy tails).
This is the regime that once left one sequence at 2.3e-3; here every sequence is checked at the
full context, in the launch configuration bench.py times:
- decode attention of all 16 sequences against the float64 oracle, latent-space and literal
  order, within 2e-3 max relative error;
- the same with sharply peaked queries built from a cached key;
- one whole sequence's K and V caches bit-exact against the oracle's quantise-and-pack of the
  GPU's own float32 latents.
"""
import math
import sys

import numpy as np
import pytest

from oracle import attention as OA, layout as OL, quant as OQ
from tests import helpers as H

pytestmark = pytest.mark.gpu

DECODE_TOL = 2e-3
FULL_SEQ = 9            # the sequence kept for the whole-cache bit-exact check


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def headline():
    import torch
    import bench
    from synth import LLAMA8B_4BIT
    _flush("[headline] preparing the bench's Llama-shaped inputs (calibrated, 1 % Student-t rows)")
    P = bench.prepare(LLAMA8B_4BIT, torch.device("cuda:0"), prefill=False, keep_latent=(FULL_SEQ,), quiet=True)
    P.host = {}
    P.upk_h, P.upv_h = bench.host_f32(P.upk), bench.host_f32(P.upv)
    yield P
    del P
    torch.cuda.empty_cache()


def _host(P, b):
    if b not in P.host:
        import bench
        P.host[b] = bench.host_seq_cache(P, b)
    return P.host[b]


def _check_all(P, q_dev, label):
    """Both decode paths on the whole batch; every sequence against the oracle."""
    import torch
    import spectral_transform_coding_amd as sp
    ctx = [P.T] * P.B
    out = sp.decode_attn(P.lay, q_dev, P.ck, P.cv, P.cap, ctx, P.upk, P.upv, P.scale)
    lit = sp.decode_attn_literal(P.lay, q_dev, P.ck, P.cv, P.cap, ctx, P.upk, P.upv, P.scale)
    torch.cuda.synchronize()
    got, got_l = out.cpu().numpy(), lit.cpu().numpy()
    q = q_dev.float().cpu().numpy().astype(np.float64)
    worst, worst_b = 0.0, -1
    for b in range(P.B):
        ck, cv = _host(P, b)
        ref = OA.decode(P.olay, q[b:b + 1], ck, cv, [P.T], P.upk_h, P.upv_h, P.scale)
        e, el = H.max_rel_err(got[b:b + 1], ref), H.max_rel_err(got_l[b:b + 1], ref)
        _flush(f"    {label} sequence {b}: latent {e:.3e}, literal {el:.3e}")
        assert e <= DECODE_TOL, (label, b, e)
        assert el <= DECODE_TOL, (label, b, el)
        if e > worst:
            worst, worst_b = e, b
    _flush(f"    {label}: worst latent-path error {worst:.3e} (sequence {worst_b})")
    return worst


@pytest.mark.timeout(900)
def test_headline_every_sequence_within_tolerance(headline):
    _check_all(headline, headline.q, "bench queries")


@pytest.mark.timeout(900)
def test_headline_peaked_queries(headline):
    # q_h proportional to the reconstructed key of one cached token per sequence (its own KV
    # head's slice), plus a little noise: attention concentrates on few tokens
    import torch
    P = headline
    rng = np.random.default_rng(77)
    dh = P.olay.d_head
    q = P.q.float().cpu().numpy().astype(np.float64)
    for b in range(P.B):
        ck, _ = _host(P, b)
        t_star = int(rng.integers(0, P.T))
        u, s = OL.read_tokens(P.olay, "K", ck, 0, np.array([t_star]))
        chat = OQ.dequantize_latent(u, s, P.olay.widths_active("K"), P.olay.g)
        kfull = OA.reconstruct(P.olay, "K", chat, P.upk_h)[0]
        for h in range(P.olay.n_q_heads):
            kv = P.olay.kv_head(h)
            k = kfull[kv * dh:(kv + 1) * dh]
            beta = 12.0 * math.sqrt(dh) / max(np.dot(k, k), 1e-12)
            q[b, h] = beta * k + 0.05 * rng.standard_normal(dh) * np.abs(k).mean()
    q_dev = torch.from_numpy(q.astype(np.float32)).cuda().to(P.q.dtype)
    _check_all(P, q_dev, "peaked")


@pytest.mark.timeout(900)
def test_headline_whole_sequence_cache_bit_exact(headline):
    P = headline
    ck, cv = _host(P, FULL_SEQ)
    ok, ov = P.olay.empty_cache("K", 1, P.cap), P.olay.empty_cache("V", 1, P.cap)
    OA.append(P.olay, ok, ov, P.lat[FULL_SEQ], 1, P.T, [0])
    for kind, got, ref in (("K", ck, ok), ("V", cv, ov)):
        if not np.array_equal(got, ref):
            bad = np.argwhere(got != ref)
            raise AssertionError(f"{kind} cache of sequence {FULL_SEQ}: {len(bad)} bytes differ, first {bad[:5].tolist()}")
    _flush(f"    sequence {FULL_SEQ}: {P.T} tokens, K and V caches bit-exact")
