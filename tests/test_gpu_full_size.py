"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The caches are written by the GPU encoder from seeded synthetic rows.  Sampled outputs are
checked against the CPU oracle, because the oracle cannot process the whole workload in test time:
- whole 128-token cache blocks, bit-exact: the oracle quantises and packs the GPU's own float32
  latent rows of those tokens into an empty cache;
- one or two sequences' decode attention, within 2e-3 max relative error, on the GPU's packed
  cache bytes.
A streaming case (append one token per sequence, then decode, repeatedly) follows the long-context
workload, once at full size with a check after the last step and once at a small size with a
check after every step.
"""
import math
import sys

import numpy as np
import pytest

from oracle import attention as OA
from synth import generators as gen
import spectral_transform_coding_amd as sp
from tests import helpers as H
from tests.test_gpu_parity import SHAPES, DECODE_TOL

pytestmark = pytest.mark.gpu

BT = 128


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Case:
    """Device caches of one workload, filled by the GPU encoder; float32 latents kept for the
    sequences that are checked."""

    def __init__(self, name, batch, cap, seed):
        import torch
        d, hq, kv, dh, ns, r, g, wk, wv, dt = SHAPES[name]
        self.olay, self.lay = H.make_layouts(d, hq, kv, dh, ns, r, g, wk, wv)
        self.dt, self.batch, self.cap, self.d = dt, batch, cap, d
        self.rng = np.random.default_rng(seed)
        self.tgen = torch.Generator(device="cuda")
        self.tgen.manual_seed(seed)
        rk, rv = self.olay.r_act("K"), self.olay.r_act("V")
        self.rk, self.rv = rk, rv
        self.w_down = H.to_dev(gen.input_dtype_round(self.rng.standard_normal((rk + rv, d)) / math.sqrt(d), dt), dt)
        # per-column spread of the hidden rows (decaying, so that latent groups differ)
        self.col_scale = torch.from_numpy((np.arange(1, d + 1, dtype=np.float32) ** -0.6) * 4.0).cuda()
        self.ck = torch.zeros(self.lay.cache_bytes(sp.TENSOR_K, batch, cap), dtype=torch.uint8, device="cuda")
        self.cv = torch.zeros(self.lay.cache_bytes(sp.TENSOR_V, batch, cap), dtype=torch.uint8, device="cuda")
        self.sk, self.sv = self.ck.numel() // batch, self.cv.numel() // batch
        self.lat = {}

    def rows(self, n):
        import torch
        x = torch.randn((n, self.d), generator=self.tgen, device="cuda", dtype=torch.float32) * self.col_scale
        return x.to(torch.bfloat16) if self.dt == "bf16" else x

    def encode(self, b, n, start, keep=False):
        """Append n new rows to sequence b at position start (one encode call)."""
        import torch
        x = self.rows(n).view(1, n, self.d)
        lat = torch.empty((n, self.rk + self.rv), dtype=torch.float32, device="cuda") if keep else None
        sp.encode_append(self.lay, x, self.w_down, self.ck[b * self.sk:(b + 1) * self.sk],
                         self.cv[b * self.sv:(b + 1) * self.sv], self.cap, [start], latent_out=lat)
        if keep:
            torch.cuda.synchronize()
            self.lat.setdefault(b, {})[start] = lat.cpu().numpy()

    def host_cache(self, b):
        """This sequence's GPU cache bytes as oracle arrays [1, blocks, block_bytes]."""
        nb = self.olay.n_blocks(self.cap)
        k = self.ck[b * self.sk:(b + 1) * self.sk].cpu().numpy().reshape(1, nb, -1)
        v = self.cv[b * self.sv:(b + 1) * self.sv].cpu().numpy().reshape(1, nb, -1)
        return k, v

    def latent_rows(self, b, t0, t1):
        """GPU float32 latent rows of tokens [t0, t1) of sequence b (from the kept calls)."""
        out = np.empty((t1 - t0, self.rk + self.rv), dtype=np.float32)
        filled = np.zeros(t1 - t0, dtype=bool)
        for start, lat in self.lat[b].items():
            lo, hi = max(t0, start), min(t1, start + lat.shape[0])
            if lo < hi:
                out[lo - t0:hi - t0] = lat[lo - start:hi - start]
                filled[lo - t0:hi - t0] = True
        assert filled.all(), "latent rows of these tokens were not kept"
        return out

    def check_blocks(self, b, blocks, ctx):
        """Cache blocks of sequence b, bit-exact against the oracle packing the GPU's latents."""
        gk, gv = self.host_cache(b)
        for blk in blocks:
            t0, t1 = blk * BT, min((blk + 1) * BT, ctx)
            ok = self.olay.empty_cache("K", 1, self.cap)
            ov = self.olay.empty_cache("V", 1, self.cap)
            OA.append(self.olay, ok, ov, self.latent_rows(b, t0, t1), 1, t1 - t0, [t0])
            for kind, got, ref in (("K", gk, ok), ("V", gv, ov)):
                if not np.array_equal(got[0, blk], ref[0, blk]):
                    bad = np.flatnonzero(got[0, blk] != ref[0, blk])
                    raise AssertionError(f"{kind} block {blk} of sequence {b}: {bad.size} bytes differ, first {bad[:8]}")

    def decode_and_check(self, ctx, check_b, seed, literal=False):
        """GPU decode of the whole batch; the listed sequences against the oracle (with
        literal=True also the literal-order decode, keys and values rebuilt then attended)."""
        import torch
        rng = np.random.default_rng(seed)
        olay, dt = self.olay, self.dt
        ups = {}
        for kind in ("K", "V"):
            rows = [H.orthonormal_rows(olay.r_act_seg(kind, s), olay.seg_cols, rng) for s in range(olay.n_seg)]
            ups[kind] = gen.input_dtype_round(np.concatenate(rows, axis=0), dt)
        q = gen.input_dtype_round(rng.standard_normal((self.batch, olay.n_q_heads, olay.d_head)), dt)
        scale = 1.0 / math.sqrt(olay.d_head)
        out = sp.decode_attn(self.lay, H.to_dev(q, dt), self.ck, self.cv, self.cap, ctx,
                             H.to_dev(ups["K"], dt), H.to_dev(ups["V"], dt), scale)
        got_lit = None
        if literal:
            lit = sp.decode_attn_literal(self.lay, H.to_dev(q, dt), self.ck, self.cv, self.cap, ctx,
                                         H.to_dev(ups["K"], dt), H.to_dev(ups["V"], dt), scale)
            torch.cuda.synchronize()
            got_lit = lit.cpu().numpy()
            del lit
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        worst = 0.0
        for b in check_b:
            hk, hv = self.host_cache(b)
            ref = OA.decode(olay, q[b:b + 1].astype(np.float64), hk, hv, [ctx[b]], ups["K"], ups["V"], scale)
            err = H.max_rel_err(got[b:b + 1], ref)
            _flush(f"    sequence {b} (ctx {ctx[b]}): max rel err {err:.3e}")
            assert err <= DECODE_TOL
            if got_lit is not None:
                err_l = H.max_rel_err(got_lit[b:b + 1], ref)
                _flush(f"    sequence {b} (ctx {ctx[b]}): literal order, max rel err {err_l:.3e}")
                assert err_l <= DECODE_TOL
                worst = max(worst, err_l)
            worst = max(worst, err)
        return worst


def test_full_c1_tiny_single_head():
    # 256-token context, one query, batch 1, fp32: everything checked
    _flush("[full] C1 tiny fp32: encode 256 tokens, decode 1 x 256")
    c = Case("tiny_f32", 1, 256, seed=21)
    c.encode(0, 256, 0, keep=True)
    c.check_blocks(0, [0, 1], 256)
    c.decode_and_check([256], [0], seed=22)


def test_full_c2_llama_prefill_and_batch16_decode():
    # encode a 32 768-token prefill per sequence, decode 16 x 32 768 (the bench's configuration)
    _flush("[full] C2 llama 4-bit: 16 x 32768")
    B, T = 16, 32768
    c = Case("llama_4bit", B, T, seed=23)
    for b in range(B):
        c.encode(b, T, 0, keep=b in (0, 11))
    c.check_blocks(0, [0, 131, 255], T)
    c.check_blocks(11, [7, 200], T)
    c.decode_and_check([T] * B, [0, 11], seed=24, literal=True)


def test_full_c3_qwen_batch32_decode():
    _flush("[full] C3 qwen 2-bit: 32 x 16384")
    B, T = 32, 16384
    c = Case("qwen_2bit", B, T, seed=25)
    for b in range(B):
        c.encode(b, T, 0, keep=b == 5)
    c.check_blocks(5, [0, 64, 127], T)
    c.decode_and_check([T] * B, [5], seed=26)


def test_full_c4_long_context_streaming():
    # decode 4 x 131 072, then 256 steps of (append one token per sequence + decode)
    import torch
    _flush("[full] C4 long context: 4 x 131072 + 256 streaming steps")
    B, T, STEPS = 4, 131072, 256
    c = Case("long_133", B, T + STEPS, seed=27)
    for b in range(B):
        c.encode(b, T, 0, keep=b == 2)
    rng = np.random.default_rng(28)
    olay, dt = c.olay, c.dt
    ups = {kind: gen.input_dtype_round(H.orthonormal_rows(olay.r_act(kind), olay.seg_cols, rng), dt)
           for kind in ("K", "V")}
    upk, upv = H.to_dev(ups["K"], dt), H.to_dev(ups["V"], dt)
    scale = 1.0 / math.sqrt(olay.d_head)
    # one workspace sized at capacity serves every step (it covers every shorter context)
    ws = torch.empty(c.lay.workspace_bytes(B, T + STEPS), dtype=torch.uint8, device="cuda")
    for step in range(STEPS):
        x = c.rows(B).view(B, 1, c.d)
        lat = torch.empty((B, c.rk + c.rv), dtype=torch.float32, device="cuda")
        sp.encode_append(c.lay, x, c.w_down, c.ck, c.cv, c.cap, [T + step] * B, latent_out=lat)
        c.lat[2][T + step] = lat[2:3].cpu().numpy()
        q = gen.input_dtype_round(rng.standard_normal((B, olay.n_q_heads, olay.d_head)), dt)
        out = sp.decode_attn(c.lay, H.to_dev(q, dt), c.ck, c.cv, c.cap, [T + step + 1] * B, upk, upv, scale,
                             workspace=ws)
    torch.cuda.synchronize()
    ctx = T + STEPS
    # the blocks the streamed tokens went to (and the prefill block before them)
    c.check_blocks(2, [T // BT - 1, T // BT, T // BT + 1], ctx)
    hk, hv = c.host_cache(2)
    ref = OA.decode(olay, q[2:3].astype(np.float64), hk, hv, [ctx], ups["K"], ups["V"], scale)
    err = H.max_rel_err(out.cpu().numpy()[2:3], ref)
    _flush(f"    after {STEPS} steps, sequence 2 (ctx {ctx}): max rel err {err:.3e}")
    assert err <= DECODE_TOL


def test_full_c5_perhead_prefill_and_batch64_decode():
    _flush("[full] C5 per-head rank 6: 64k prefill encode; decode 64 x 32768")
    pre = Case("perhead_r6", 1, 65536, seed=29)
    pre.encode(0, 65536, 0, keep=True)
    pre.check_blocks(0, [0, 255, 511], 65536)
    B, T = 64, 32768
    c = Case("perhead_r6", B, T, seed=30)
    for b in range(B):
        c.encode(b, T, 0, keep=b == 17)
    c.check_blocks(17, [3, 250], T)
    c.decode_and_check([T] * B, [17], seed=31)


def test_streaming_append_then_decode_every_step():
    # the long-context workload's streaming pattern at a small size, checked after every step:
    # caches bit-exact against the oracle's appends, decode against the oracle's attention
    import torch
    _flush("[stream] long_133 small: 8 steps")
    B, cap = 3, 640
    c = Case("long_133", B, cap, seed=32)
    olay, dt = c.olay, c.dt
    ctx = [300, 37, 129]
    ok, ov = olay.empty_cache("K", B, cap), olay.empty_cache("V", B, cap)
    for b in range(B):
        c.encode(b, ctx[b], 0, keep=True)
        OA.append(olay, ok[b:b + 1], ov[b:b + 1], c.latent_rows(b, 0, ctx[b]), 1, ctx[b], [0])
    rng = np.random.default_rng(33)
    ups = {kind: gen.input_dtype_round(H.orthonormal_rows(olay.r_act(kind), olay.seg_cols, rng), dt)
           for kind in ("K", "V")}
    upk, upv = H.to_dev(ups["K"], dt), H.to_dev(ups["V"], dt)
    scale = 1.0 / math.sqrt(olay.d_head)
    for step in range(8):
        x = c.rows(B).view(B, 1, c.d)
        lat = torch.empty((B, c.rk + c.rv), dtype=torch.float32, device="cuda")
        sp.encode_append(c.lay, x, c.w_down, c.ck, c.cv, cap, ctx, latent_out=lat)
        torch.cuda.synchronize()
        OA.append(olay, ok, ov, lat.cpu().numpy(), B, 1, ctx)
        ctx = [t + 1 for t in ctx]
        gk = c.ck.cpu().numpy().reshape(ok.shape)
        gv = c.cv.cpu().numpy().reshape(ov.shape)
        assert np.array_equal(gk, ok) and np.array_equal(gv, ov), f"caches differ after step {step}"
        q = gen.input_dtype_round(rng.standard_normal((B, olay.n_q_heads, olay.d_head)), dt)
        out = sp.decode_attn(c.lay, H.to_dev(q, dt), c.ck, c.cv, cap, ctx, upk, upv, scale)
        torch.cuda.synchronize()
        ref = OA.decode(olay, q.astype(np.float64), ok, ov, ctx, ups["K"], ups["V"], scale)
        err = H.max_rel_err(out.cpu().numpy(), ref)
        assert err <= DECODE_TOL, (step, err)
    _flush(f"    8 steps: caches bit-exact, last max rel err {err:.3e}")
