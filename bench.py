#!/usr/bin/env python3
"""Benchmark of the latent KV codec's hot path on one MI355X.

One timed step = one pass of the whole path over one batch of synthetic input, for the
Llama-3.1-8B-shaped layer (hidden 4096, 32 query heads, 8 KV heads, d_head 128, latent rank
512 per tensor, groups of 16, 4 bits per element with scales):
  encode: spectra_encode_append of one 32 768-token prefill (down-projection GEMM on the
          matrix cores, per-token group quantisation, bit-packing, append);
  decode: spectra_decode_attn for batch 16 x 32 768 context, one query token each.
Inputs are generated on the GPU before timing and stay resident in HBM.  The decode caches
rotate over copies of at least 1 GiB in all, so that no step finds its cache in the 256 MB
Infinity Cache ("cold").  During the timed steps the library records HIP events around the
decode's streaming kernel on its own stream; the roofline figure comes from those.

The four other workloads are measured after the timed steps, each at its full size, and are
reported under "workloads": the tiny fp32 head (latency, microseconds), the Qwen-shaped 2-bit
layer (cold decode), the 128k long-context 4/3-bit layer (cold decode, then 256 steps of a
one-token append per sequence and a decode), and the per-head rank-6 layer (64k-token prefill
encode against HBM, cold decode).  Each carries the CPU oracle's rates on bounded samples of
the same workload (calibration, encode, decode).

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix
COLD_BYTES = 1 << 30           # cache copies rotated per decode measurement
KERNEL_EVERY = 4               # timed steps with library events around the stream kernel: one in four


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- host info

def cpu_info():
    """(CPU model string, BLAS threads the oracle runs with)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    return model, int(threads)


# ------------------------------------------------------------------------- workload inputs

class Prepared:
    """One workload's resident device inputs (see prepare)."""


def _calibrate(sp, wl, G, wk, wv):
    if wl.fixed_width:
        return sp.calibrate(G, wk, wv, wl.n_kv_heads, wl.d_head, wl.n_seg, wl.seg_rank, wl.group_size,
                            fixed_width=wl.fixed_width, energy=wl.energy or 0.0)
    return sp.calibrate(G, wk, wv, wl.n_kv_heads, wl.d_head, wl.n_seg, wl.seg_rank, wl.group_size,
                        wl.budget_bits)


def prepare(wl, dev, prefill=True, keep_latent=(), batch=None, ctx=None, quiet=False):
    """Calibrates the workload on device-drawn rows (G on the GPU, spectra_calibrate on the
    host), fills its decode caches with the GPU encoder and draws its queries.
    keep_latent: sequences whose float32 latents (encode's test hook) are kept on the host.
    Returns a Prepared with lay/olay, cal, G, wk/wv/wq, w_down_t/upk/upv (device), ck/cv,
    q (device), B, T, cap, scale, x_pre/pre_k/pre_v (prefill, if asked), lat {b: array}."""
    import numpy as np
    import torch
    import spectral_transform_coding_amd as sp
    from synth import generators as gen
    from oracle import layout as OL
    say = (lambda m: None) if quiet else log
    P = Prepared()
    P.wl = wl
    d, hq, kv, dh = wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.d_head
    try:
        Q = gen.basis_torch(wl, dev)
    except Exception as e:            # data generation only
        say(f"device QR unavailable ({e}); drawing the basis on the host")
        Q = torch.from_numpy(gen.basis(wl).astype(np.float32)).to(dev)
    P.Q = Q
    G = torch.zeros((d, d), dtype=torch.float64, device=dev)
    for c0 in range(0, wl.calib_rows, 4096):
        h = gen.hidden_rows_torch(wl, min(4096, wl.calib_rows - c0), 200000 + c0 // 4096, Q, dev).double()
        G += h.T @ h
    P.G = (G / wl.calib_rows).cpu().numpy()
    del G
    P.wk, P.wv, P.wq, P.wo = gen.projection_weights(wl)
    t0 = time.perf_counter()
    P.cal = _calibrate(sp, wl, P.G, P.wk, P.wv)
    P.calibrate_s = time.perf_counter() - t0
    say(f"{wl.name}: calibrate {P.calibrate_s:.1f} s, widths K {P.cal['widths_k'].reshape(-1).tolist()}")
    P.lay = sp.Layout(d, hq, kv, dh, wl.n_seg, wl.seg_rank, wl.group_size, P.cal["widths_k"], P.cal["widths_v"])
    P.olay = OL.Layout(d, hq, kv, dh, wl.n_seg, wl.seg_rank, wl.group_size, P.cal["widths_k"], P.cal["widths_v"])
    P.tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(P.tdt)
    P.w_down_t = dv(np.concatenate([P.cal["w_down_t_k"], P.cal["w_down_t_v"]], axis=0))
    P.upk, P.upv = dv(P.cal["w_up_k"]), dv(P.cal["w_up_v"])
    P.rk, P.rv = P.cal["r_act_k"], P.cal["r_act_v"]
    P.B = wl.decode_batch if batch is None else batch
    P.T = wl.decode_ctx if ctx is None else ctx
    P.cap = P.T + wl.stream_steps
    P.scale = 1.0 / math.sqrt(dh)
    P.ck = torch.zeros(P.lay.cache_bytes(0, P.B, P.cap), dtype=torch.uint8, device=dev)
    P.cv = torch.zeros(P.lay.cache_bytes(1, P.B, P.cap), dtype=torch.uint8, device=dev)
    P.sk, P.sv = P.ck.numel() // P.B, P.cv.numel() // P.B
    P.lat = {}
    for b in range(P.B):
        xb = gen.hidden_rows_torch(wl, P.T, 101 + b, Q, dev).to(P.tdt).view(1, P.T, d)
        lat = torch.empty((P.T, P.rk + P.rv), dtype=torch.float32, device=dev) if b in keep_latent else None
        sp.encode_append(P.lay, xb, P.w_down_t, P.ck[b * P.sk:(b + 1) * P.sk], P.cv[b * P.sv:(b + 1) * P.sv],
                         P.cap, [0], latent_out=lat)
        if lat is not None:
            P.lat[b] = lat.cpu().numpy()
        del xb
    hq_rows = gen.hidden_rows_torch(wl, P.B, gen.STREAM_QUERY, Q, dev)
    P.q = (hq_rows.double() @ torch.from_numpy(P.wq).to(dev)).view(P.B, hq, dh).to(P.tdt)
    if prefill:
        n = wl.encode_tokens
        P.x_pre = gen.hidden_rows_torch(wl, n, 100, Q, dev).to(P.tdt).view(1, n, d)
        P.pre_k = torch.zeros(P.lay.cache_bytes(0, 1, n), dtype=torch.uint8, device=dev)
        P.pre_v = torch.zeros(P.lay.cache_bytes(1, 1, n), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return P


def cache_bytes_per_call(P, ctx):
    """Packed cache bytes a decode over contexts `ctx` streams (codes and scales of K and V)."""
    per_tok = (P.lay.block_bytes(0) + P.lay.block_bytes(1)) / 128.0
    return per_tok * float(sum(ctx))


def small_bytes(P):
    """q, W_up (both tensors) and the float32 output: read or written once per decode call."""
    return P.q.numel() * P.q.element_size() + (P.upk.numel() + P.upv.numel()) * P.upk.element_size() + \
        P.B * P.wl.n_q_heads * P.wl.d_head * 4


def cold_copies(P, min_bytes=COLD_BYTES):
    """The caches and clones of them, at least min_bytes in all (at least two copies)."""
    per = P.ck.numel() + P.cv.numel()
    n = max(2, -(-min_bytes // per))
    return [(P.ck, P.cv)] + [(P.ck.clone(), P.cv.clone()) for _ in range(n - 1)]


def kernel_step(i, steps):
    """Whether timed step i records the library's events around the stream kernel (one step in
    KERNEL_EVERY, and the last step of a shorter run)."""
    return i % KERNEL_EVERY == KERNEL_EVERY - 1 or (steps < KERNEL_EVERY and i == steps - 1)


def new_events(n, k):
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(k)] for _ in range(n)]
    for e in evs:                   # create the HIP events before handing them to the library
        for ev in e:
            ev.record()
    torch.cuda.synchronize()
    return evs


def head_start(ms):
    """A bounded sleep kernel of about `ms` milliseconds enqueued ahead of a timing loop, so that
    the host queues the loop's calls while the GPU is busy and the events then time the GPU's own
    back-to-back execution, not the rate at which Python enqueues (latency-bound calls take less
    GPU time than their host-side launch)."""
    import torch
    try:
        torch.cuda._sleep(int(ms * 2.4e6))
    except Exception:            # timing only: without it the loop may be paced by the host
        pass


def time_decode(P, copies, calls, warmup=3):
    """Mean decode-call time and mean stream-kernel time, in ms, over `calls` calls rotating
    `copies`.  As in the headline steps, the call time comes from the calls without the
    library's kernel events (events around the call only) and the kernel time from the calls
    with them (one call in KERNEL_EVERY): the two extra event records inside a call add a few
    microseconds to it."""
    import numpy as np
    import torch
    import spectral_transform_coding_amd as sp
    ctx = [P.T] * P.B
    ws = torch.empty(max(P.lay.workspace_bytes(P.B, P.T), 1), dtype=torch.uint8, device=P.q.device)
    out = torch.empty((P.B, P.wl.n_q_heads, P.wl.d_head), dtype=torch.float32, device=P.q.device)
    for i in range(warmup):
        ck, cv = copies[i % len(copies)]
        sp.decode_attn(P.lay, P.q, ck, cv, P.cap, ctx, P.upk, P.upv, P.scale, out=out, workspace=ws)
    evs = new_events(calls, 4)
    head_start(0.25 * calls)
    for i in range(calls):
        ck, cv = copies[i % len(copies)]
        if kernel_step(i, calls):
            sp.set_timing_events(evs[i][1], evs[i][2])
        evs[i][0].record()
        sp.decode_attn(P.lay, P.q, ck, cv, P.cap, ctx, P.upk, P.upv, P.scale, out=out, workspace=ws)
        evs[i][3].record()
    torch.cuda.synchronize()
    plain = [e[0].elapsed_time(e[3]) for i, e in enumerate(evs) if not kernel_step(i, calls)]
    call = float(np.mean(plain if plain else [e[0].elapsed_time(e[3]) for e in evs]))
    kern = float(np.mean([e[1].elapsed_time(e[2]) for i, e in enumerate(evs) if kernel_step(i, calls)]))
    assert torch.isfinite(out).all().item(), "non-finite decode output"
    return call, kern, out


def time_encode(P, calls, warmup=2):
    """Mean time (ms) of one prefill encode call (one kernel) on the resident prefill rows.  Every
    call re-encodes the same rows into the same positions (the ORed words then receive the bits
    they already hold), as the timed steps do."""
    import numpy as np
    import torch
    import spectral_transform_coding_amd as sp
    n = P.x_pre.shape[1]
    for _ in range(warmup):
        sp.encode_append(P.lay, P.x_pre, P.w_down_t, P.pre_k, P.pre_v, n, [0])
    evs = new_events(calls, 2)
    head_start(0.15 * calls)
    for i in range(calls):
        evs[i][0].record()
        sp.encode_append(P.lay, P.x_pre, P.w_down_t, P.pre_k, P.pre_v, n, [0])
        evs[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))


def rel_err(o, r):
    """max over heads of |o - r|_inf / |r|_inf (both [Hq, d_head])."""
    import numpy as np
    return float(np.max(np.abs(o - r).max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-300)))


# ------------------------------------------------------------------------ CPU oracle timing

def host_seq_cache(P, b):
    ck = P.ck[b * P.sk:(b + 1) * P.sk].view(-1, P.lay.block_bytes(0)).cpu().numpy()[None]
    cv = P.cv[b * P.sv:(b + 1) * P.sv].view(-1, P.lay.block_bytes(1)).cpu().numpy()[None]
    return ck, cv


def host_f32(t):
    return t.float().cpu().numpy()


def cpu_decode(P, target_s):
    """The oracle's decode (float64 NumPy) on a growing prefix of sequence 0 until about target_s
    of CPU work.  Returns (GB/s of packed cache, tokens, seconds, output if the whole sequence
    was done else None)."""
    import numpy as np
    from oracle import attention as OA
    ck, cv = host_seq_cache(P, 0)
    q = host_f32(P.q[:1]).astype(np.float64)
    upk, upv = host_f32(P.upk), host_f32(P.upv)
    per_tok = (P.lay.block_bytes(0) + P.lay.block_bytes(1)) / 128.0
    n = min(P.T, 1024)
    while True:
        t0 = time.perf_counter()
        ref = OA.decode(P.olay, q, ck, cv, [n], upk, upv, P.scale)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= P.T:
            break
        n = min(P.T, max(n * 2, int(n * target_s / max(dt, 1e-3) * 1.1)) // 128 * 128)
    return n * per_tok / dt / 1e9, n, dt, (ref if n == P.T else None)


def cpu_encode(P, target_s):
    """The oracle's encode (float64 projection, float32 latent, quantise and pack) of a growing
    number of the prefill's rows.  Returns (tokens/s, tokens, seconds)."""
    import numpy as np
    from oracle import attention as OA
    xs = host_f32(P.x_pre[0, :min(P.x_pre.shape[1], 65536)])
    w = host_f32(P.w_down_t).T
    n = min(xs.shape[0], 128)
    while True:
        ok, ov = P.olay.empty_cache("K", 1, n), P.olay.empty_cache("V", 1, n)
        t0 = time.perf_counter()
        lat = OA.encode_latent(xs[:n], w).astype(np.float32)
        OA.append(P.olay, ok, ov, lat, 1, n, [0])
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= xs.shape[0]:
            break
        n = min(xs.shape[0], max(n * 2, int(n * target_s / max(dt, 1e-3) * 1.1)))
    return n / dt, n, dt


def cpu_calibrate(P):
    """Seconds the oracle's calibration (G-weighted eigen-decomposition, water-filling) takes on
    the same G and weights."""
    from oracle import calibrate as OC
    wl = P.wl
    t0 = time.perf_counter()
    if wl.fixed_width:
        OC.calibrate(P.G, P.wk, P.wv, wl.n_seg, wl.seg_rank, wl.group_size, 0.0, fixed_width=wl.fixed_width,
                     energy=wl.energy)
    else:
        OC.calibrate(P.G, P.wk, P.wv, wl.n_seg, wl.seg_rank, wl.group_size, wl.budget_bits)
    return time.perf_counter() - t0


def cpu_record(P, decode_s, encode_s, with_encode):
    model, threads = cpu_info()
    gbs, n, dt, _ = cpu_decode(P, decode_s)
    rec = {"kind": "oracle", "cores": threads, "cpu": model,
           "decode_GB_s": round(gbs, 6),
           "decode_sample": f"1 sequence x {n} tokens x {P.wl.n_q_heads} heads in {dt:.2f} s",
           "calibrate_s": round(cpu_calibrate(P), 3)}
    if with_encode:
        tps, ne, dte = cpu_encode(P, encode_s)
        rec["encode_tok_s"] = round(tps, 2)
        rec["encode_sample"] = f"{ne} tokens in {dte:.2f} s"
    return rec


# ----------------------------------------------------------------------------- measurements

def measured_profile_field(name, field, sources):
    """An integer field of a committed rocprofv3 summary in profiles/, or None when the named
    sources have changed since it was taken (their sha256 is recorded in the summary)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    try:
        fields = dict(l.split(":", 1) for l in open(path) if l[:1] not in "# " and ":" in l)
    except OSError:
        return None
    src = os.path.join(ROOT, "spectral_transform_coding_amd", "csrc")
    h = hashlib.sha256(b"".join(open(os.path.join(src, n), "rb").read() for n in sources))
    if h.hexdigest() != fields.get("source_sha256", "").strip() or field not in fields:
        return None
    return float(fields[field])


DECODE_SOURCES = ("spectra_decode_mfma.h", "spectra_decode.hip", "spectra_device.h", "spectra_internal.h")
ENCODE_SOURCES = ("spectra_encode.hip", "spectra_device.h", "spectra_internal.h")


def copy_only(args):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))


def headline(args, dev):
    """The timed steps on the Llama-shaped workload.  Returns (result dict, Prepared)."""
    import numpy as np
    import torch
    import spectral_transform_coding_amd as sp
    from synth import LLAMA8B_4BIT as wl
    P = prepare(wl, dev)
    B, T, NPRE = P.B, P.T, wl.encode_tokens
    copies = cold_copies(P)
    ctx = [T] * B
    ws = torch.empty(P.lay.workspace_bytes(B, T), dtype=torch.uint8, device=dev)
    out = torch.empty((B, wl.n_q_heads, wl.d_head), dtype=torch.float32, device=dev)

    def step(i, evs=None):
        ck_i, cv_i = copies[i % len(copies)]
        if evs:
            evs[0].record()
        sp.encode_append(P.lay, P.x_pre, P.w_down_t, P.pre_k, P.pre_v, NPRE, [0])
        if evs:
            evs[1].record()
            if kernel_step(i, args.steps):
                sp.set_timing_events(evs[2], evs[3])
        sp.decode_attn(P.lay, P.q, ck_i, cv_i, P.cap, ctx, P.upk, P.upv, P.scale, out=out, workspace=ws)
        if evs:
            evs[4].record()

    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item(), "non-finite decode output"
    events = new_events(args.steps, 5)
    log(f"timing {args.steps} steps ({len(copies)} cache copies, {len(copies) * (P.ck.numel() + P.cv.numel()) / 1e9:.2f} GB)")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    # the call time from the steps without library events (two event records inside the call
    # add a few microseconds), the stream kernel's from the steps with them
    plain = [e[1].elapsed_time(e[4]) for i, e in enumerate(events) if not kernel_step(i, args.steps)]
    dec_ms = float(np.mean(plain if plain else [e[1].elapsed_time(e[4]) for e in events]))
    strm_ms = float(np.mean([e[2].elapsed_time(e[3]) for i, e in enumerate(events) if kernel_step(i, args.steps)]))
    ms_step = (t1 - t0) * 1e3 / args.steps
    cbytes = cache_bytes_per_call(P, ctx)
    dec_bytes = cbytes + small_bytes(P)
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    strm_gbs = cbytes / (strm_ms * 1e-3) / 1e9
    enc_flop = 2.0 * NPRE * wl.d_model * (P.rk + P.rv)
    enc_tflops = enc_flop / (enc_ms * 1e-3) / 1e12
    log(f"encode {enc_ms:.3f} ms ({NPRE / enc_ms / 1e3:.1f} Mtok/s, {enc_tflops:.0f} TFLOP/s); "
        f"decode {dec_ms:.3f} ms ({dec_gbs:.0f} GB/s), stream kernel {strm_ms:.3f} ms ({strm_gbs:.0f} GB/s)")
    mfma_busy = measured_profile_field("encode_llama8b_prefill32768_mfma_busy.txt", "mfma_busy_frac", ENCODE_SOURCES)
    res = {
        "metric": "latent-KV decode-attn achieved HBM GB/s (% peak); encode Mtok/s at 1 GPU",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs; f16 matrix-core products with f32 accumulation; u1-u8 codes",
        "data": "synthetic (seeded Gaussian rows with i^-1.2 eigen-decay and 1% Student-t(3) rows, random weights)",
        "config": {"workload": wl.name, "d_model": wl.d_model, "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "d_head": wl.d_head, "latent_rank": wl.seg_rank, "group_size": wl.group_size,
                   "budget_bits": wl.budget_bits, "decode_batch": B, "decode_ctx": T, "encode_tokens": NPRE,
                   "bytes_per_token_kv": round(cbytes / (B * T), 2), "cache_copies": len(copies)},
        "decode": {"ms": round(dec_ms, 4), "GB_s": round(dec_gbs, 1), "pct_peak": round(100 * dec_gbs / PEAK_HBM_GBS, 2),
                   "algorithmic_bytes": int(dec_bytes), "cold": True},
        "encode": {"ms": round(enc_ms, 4), "Mtok_s": round(NPRE / enc_ms / 1e3, 2), "TFLOP_s": round(enc_tflops, 1),
                   "mfma_frac": round(enc_tflops / PEAK_BF16_TFLOPS, 4), "mfma_busy_rocprof": mfma_busy},
        "roofline": {"kernel": "spectra_decode_jit (decode stream kernel)", "bound": "hbm", "achieved": round(strm_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(strm_gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_profile_field("decode_llama8b_b16_ctx32768_hbm_counters.txt",
                                                       "traffic_bytes_per_launch", DECODE_SOURCES),
                     "algorithmic_bytes_per_launch": int(cbytes), "avg_launch_ms": round(strm_ms, 4),
                     "timing": "HIP events attached by the library to the kernel's own dispatch "
                               "(hipExtModuleLaunchKernel), in one of every four timed steps"},
        "calibrate_s": round(P.calibrate_s, 2),
    }
    P.out = out
    P.ws = ws
    del copies
    return res, P


def literal_compare(P, dev, n=5):
    """The literal-order call (keys and values rebuilt, then attended) on the same inputs."""
    import numpy as np
    import torch
    import spectral_transform_coding_amd as sp
    ctx = [P.T] * P.B
    lit_ws = torch.empty(P.lay.literal_workspace_bytes(P.B, P.T), dtype=torch.uint8, device=dev)
    lit_out = torch.empty_like(P.out)
    for _ in range(2):
        sp.decode_attn_literal(P.lay, P.q, P.ck, P.cv, P.cap, ctx, P.upk, P.upv, P.scale, out=lit_out, workspace=lit_ws)
    evs = new_events(n, 2)
    for i in range(n):
        evs[i][0].record()
        sp.decode_attn_literal(P.lay, P.q, P.ck, P.cv, P.cap, ctx, P.upk, P.upv, P.scale, out=lit_out, workspace=lit_ws)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sp.decode_attn(P.lay, P.q, P.ck, P.cv, P.cap, ctx, P.upk, P.upv, P.scale, out=P.out, workspace=P.ws)
    torch.cuda.synchronize()
    dmat = (lit_out - P.out).abs().amax(dim=2) / P.out.abs().amax(dim=2).clamp_min(1e-30)
    P.lit_out = lit_out
    return {"ms": round(ms, 4), "max_rel_diff_vs_latent": float(f"{float(dmat.max()):.3e}"),
            "max_diff_sequence": int(dmat.amax(dim=1).argmax()), "calls": n}


def oracle_check(P, seqs, lit=False):
    """Sampled check: decode of the listed sequences (whole contexts) against the oracle."""
    import numpy as np
    from oracle import attention as OA
    checks = []
    for b in seqs:
        ck, cv = host_seq_cache(P, b)
        ref = OA.decode(P.olay, host_f32(P.q[b:b + 1]).astype(np.float64), ck, cv, [P.T], host_f32(P.upk),
                        host_f32(P.upv), P.scale)[0]
        chk = {"sequence": int(b), "tokens": P.T, "latent_max_rel_err": float(f"{rel_err(host_f32(P.out[b]), ref):.3e}")}
        if lit:
            chk["literal_max_rel_err"] = float(f"{rel_err(host_f32(P.lit_out[b]), ref):.3e}")
        log(f"oracle check {P.wl.name}: {chk}")
        checks.append(chk)
    return checks


def decode_record(P, call_ms, kern_ms, copies, kernel):
    cb = cache_bytes_per_call(P, [P.T] * P.B)
    gbs = (cb + small_bytes(P)) / (call_ms * 1e-3) / 1e9
    kgbs = cb / (kern_ms * 1e-3) / 1e9
    return {"batch": P.B, "ctx": P.T, "ms": round(call_ms, 4), "GB_s": round(gbs, 1),
            "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "cache_bytes": int(cb),
            "cold": len(copies) * (P.ck.numel() + P.cv.numel()) >= COLD_BYTES, "copies": len(copies),
            "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4), "avg_launch_ms": round(kern_ms, 4)}}


def extra_workloads(args, dev, names):
    """Measurements of the other four workloads at full size (see the module docstring)."""
    import numpy as np
    import torch
    import spectral_transform_coding_amd as sp
    from synth import TINY, QWEN7B_2BIT, LLAMA8B_LONG, PERHEAD_R6
    out = {}
    for wl in (TINY, QWEN7B_2BIT, LLAMA8B_LONG, PERHEAD_R6):
        if names and wl.name not in names:
            continue
        log(f"workload {wl.name}")
        rec = {}
        P = prepare(wl, dev, prefill=wl.name in (TINY.name, PERHEAD_R6.name))
        if wl is TINY:
            # latency-bound: 8 KB of cache; the call time is the figure (microseconds)
            copies = [(P.ck, P.cv)]
            call, kern, o = time_decode(P, copies, 200)
            enc = time_encode(P, 200)
            rec["decode"] = {"batch": P.B, "ctx": P.T, "us": round(call * 1e3, 2), "kernel_us": round(kern * 1e3, 2),
                             "kind": "latency (cache resident)"}
            rec["encode"] = {"tokens": wl.encode_tokens, "us": round(enc * 1e3, 2)}
            P.out = o
            rec["oracle_check"] = oracle_check(P, [0])
        else:
            copies = cold_copies(P)
            call, kern, o = time_decode(P, copies, args.calls)
            # per-head layout: the one-launch small-rank kernel (absorption, stream, merge, lift)
            kernel = "decode_small_fused_kernel" if wl.n_seg > 1 else "spectra_decode_jit"
            rec["decode"] = decode_record(P, call, kern, copies, kernel)
            log(f"  decode {call * 1e3:.1f} us ({rec['decode']['GB_s']} GB/s cold), stream kernel {kern * 1e3:.1f} us "
                f"({rec['decode']['roofline']['frac'] * 100:.1f} % of HBM)")
            del copies
        if wl is PERHEAD_R6:
            enc = time_encode(P, 20)
            n = wl.encode_tokens
            ebytes = P.x_pre.numel() * P.x_pre.element_size() + P.w_down_t.numel() * P.w_down_t.element_size() + \
                n * (P.lay.block_bytes(0) + P.lay.block_bytes(1)) / 128.0
            egbs = ebytes / (enc * 1e-3) / 1e9
            rec["encode"] = {"tokens": n, "ms": round(enc, 4), "Mtok_s": round(n / enc / 1e3, 2),
                             "roofline": {"kernel": "encode_mfma_kernel", "bound": "hbm", "achieved": round(egbs, 1),
                                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(egbs / PEAK_HBM_GBS, 4),
                                          "algorithmic_bytes": int(ebytes)}}
            log(f"  encode {n} tokens {enc:.3f} ms ({egbs:.0f} GB/s)")
        if wl is LLAMA8B_LONG and not args.no_streaming:
            rec["stream_steps"] = streaming(P, dev)
        if not args.no_cpu_baseline:
            rec["cpu_oracle"] = cpu_record(P, 2.0 if wl is not TINY else 0.2, 2.0, wl in (TINY, PERHEAD_R6))
        out[wl.name] = rec
        del P
        torch.cuda.empty_cache()
    return out


def streaming(P, dev):
    """256 steps of (append one token per sequence, decode over everything so far), the long-
    context workload's serving pattern.  The cache stays the same buffer (it fits the 256 MB
    Infinity Cache, so this loop is "hot").  Per-step times from events."""
    import numpy as np
    import torch
    import spectral_transform_coding_amd as sp
    from synth import generators as gen
    wl, B, T = P.wl, P.B, P.T
    steps = wl.stream_steps
    x = gen.hidden_rows_torch(wl, steps * B, 10 ** 6, P.Q, dev).to(P.tdt).view(steps, B, 1, wl.d_model)
    ws = torch.empty(P.lay.workspace_bytes(B, T + steps), dtype=torch.uint8, device=dev)
    out = torch.empty((B, wl.n_q_heads, wl.d_head), dtype=torch.float32, device=dev)
    evs = new_events(steps, 3)
    torch.cuda.synchronize()
    head_start(0.4 * steps)
    for s in range(steps):
        evs[s][0].record()
        sp.encode_append(P.lay, x[s], P.w_down_t, P.ck, P.cv, P.cap, [T + s] * B)
        evs[s][1].record()
        sp.decode_attn(P.lay, P.q, P.ck, P.cv, P.cap, [T + s + 1] * B, P.upk, P.upv, P.scale, out=out, workspace=ws)
        evs[s][2].record()
    torch.cuda.synchronize()
    app = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    cb = cache_bytes_per_call(P, [T + steps // 2] * B)
    log(f"  streaming: append {app * 1e3:.1f} us + decode {dec * 1e3:.1f} us per step (GPU)")
    return {"steps": steps, "append_us": round(app * 1e3, 2), "decode_us": round(dec * 1e3, 2),
            "us_per_step": round((app + dec) * 1e3, 2),
            "decode_GB_s": round(cb / (dec * 1e-3) / 1e9, 1), "cold": False}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400, help="timed headline steps (encode + decode)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--calls", type=int, default=200, help="timed decode calls per extra workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-only", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="skip the four other workloads")
    ap.add_argument("--workloads", default="", help="comma-separated names of the other workloads to run")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip the long-context workload's 256-step append + decode loop")
    ap.add_argument("--skip-headline", action="store_true",
                    help="run only the other workloads (per-workload profiles); the line then has no headline figures")
    ap.add_argument("--no-literal", action="store_true",
                    help="skip the literal-order decode (keys and values rebuilt, then attended)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library drives one "
              "device per process and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_only:
        return copy_only(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.skip_headline:
        names = [s for s in args.workloads.split(",") if s]
        print(json.dumps({"workloads": extra_workloads(args, dev, names)}), flush=True)
        return
    res, P = headline(args, dev)
    if not args.no_literal:
        log("literal-order decode")
        lit = literal_compare(P, dev)
        lit["x_latent_call"] = round(lit["ms"] / res["decode"]["ms"], 2)
        res["literal_decode"] = lit
        log(f"literal-order decode {lit['ms']:.3f} ms ({lit['x_latent_call']}x the latent-space call)")
    if not args.no_cpu_baseline:
        log("CPU baseline (oracle) and sampled oracle check")
        model, threads = cpu_info()
        gbs, n, dt, ref0 = cpu_decode(P, 6.0)
        bpt = (P.lay.block_bytes(0) + P.lay.block_bytes(1)) / 128.0
        res["cpu_baseline"] = {"value": round(gbs, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
                               "cpu": model,
                               "sample": f"float64 NumPy oracle decode of 1 sequence x {n} tokens x "
                                         f"{P.wl.n_q_heads} heads ({n * bpt / 1e6:.1f} MB packed cache) in {dt:.2f} s"}
        tps, ne, dte = cpu_encode(P, 3.0)
        res["cpu_baseline"]["encode_tok_s"] = round(tps, 2)
        res["cpu_baseline"]["encode_sample"] = f"{ne} prefill tokens (projection, quantise, pack) in {dte:.2f} s"
        res["cpu_baseline"]["calibrate_s"] = round(cpu_calibrate(P), 3)
        seqs = [0]
        if "literal_decode" in res:
            seqs.append(res["literal_decode"]["max_diff_sequence"])
        seqs.append(9)
        chks = oracle_check(P, sorted(set(seqs)), lit="literal_decode" in res)
        res["oracle_check"] = {"sampled": True, "tol": 2e-3, "sequences": chks,
                               "within_tol": all(c["latent_max_rel_err"] <= 2e-3 for c in chks)}
    del P
    torch.cuda.empty_cache()
    if not args.headline_only:
        names = [s for s in args.workloads.split(",") if s]
        res["workloads"] = extra_workloads(args, dev, names)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
