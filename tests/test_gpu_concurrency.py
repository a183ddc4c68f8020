"""Decode calls from several host threads at once, each on its own stream with its own output and
workspace, on a layout whose specialised kernel has not been compiled yet: the threads may compile
it concurrently (the library keeps the first module to finish and unloads the others). Every
thread's output must equal, bit for bit, the width-generic kernel's output for the same inputs
(the specialised kernel computes the same arithmetic in the same order), and so must a later call
that finds the kernel in the cache."""
import math
import sys
import threading

import numpy as np
import pytest

from synth import generators as gen
import spectral_transform_coding_amd as sp
from tests import helpers as H

pytestmark = pytest.mark.gpu

# widths used by no other test, so the first call in the process compiles the specialised kernel
WK = [8, 6, 6, 5, 5, 4, 4, 3, 3, 3, 2, 2, 2, 1, 1, 1]
WV = [7, 7, 5, 5, 4, 4, 4, 3, 3, 2, 2, 2, 1, 1, 0, 0]
N_THREADS = 4


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_concurrent_first_calls_share_one_specialised_kernel():
    import torch
    _flush(f"[concurrency] {N_THREADS} threads, first decode of a new layout")
    d, hq, kv, dh, r, dt = 1024, 16, 4, 64, 256, "bf16"
    olay, lay = H.make_layouts(d, hq, kv, dh, 1, r, 16, WK, WV)
    rng = np.random.default_rng(71)
    ctx, cap = [1500, 77, 1024, 0, 640], 1536
    B = len(ctx)
    ck, cv, _ = H.build_caches(olay, B, cap, ctx, rng, outlier_frac=0.01)
    ups = {}
    for kind in ("K", "V"):
        ups[kind] = H.to_dev(gen.input_dtype_round(H.orthonormal_rows(olay.r_act_seg(kind, 0), olay.seg_cols, rng), dt), dt)
    q = H.to_dev(gen.input_dtype_round(rng.standard_normal((B, hq, dh)), dt), dt)
    dck, dcv = H.dev_bytes(ck), H.dev_bytes(cv)
    scale = 1.0 / math.sqrt(dh)

    prev = sp.set_jit(0)
    try:
        generic = sp.decode_attn(lay, q, dck, dcv, cap, ctx, ups["K"], ups["V"], scale)
        torch.cuda.synchronize()
    finally:
        sp.set_jit(1)
    try:
        assert np.isfinite(generic.cpu().numpy()).all()
        wsb = max(lay.workspace_bytes(B, cap), 1)
        outs = [torch.full_like(generic, float("nan")) for _ in range(N_THREADS)]
        wss = [torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(N_THREADS)]
        streams = [torch.cuda.Stream() for _ in range(N_THREADS)]
        torch.cuda.synchronize()
        n_kernels = sp.jit_kernel_count()
        start = threading.Barrier(N_THREADS)
        errors = []

        def run(i):
            try:
                start.wait(timeout=60)
                with torch.cuda.stream(streams[i]):
                    sp.decode_attn(lay, q, dck, dcv, cap, ctx, ups["K"], ups["V"], scale,
                                   out=outs[i], workspace=wss[i], stream=streams[i])
                streams[i].synchronize()
            except Exception as e:                      # reported by the main thread
                errors.append(f"thread {i}: {e!r}")

        threads = [threading.Thread(target=run, args=(i,)) for i in range(N_THREADS)]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=100)
        assert not any(t.is_alive() for t in threads), "a decode thread did not finish"
        assert not errors, errors
        torch.cuda.synchronize()
        # one module kept for the layout, whichever threads compiled it
        assert sp.jit_kernel_count() == n_kernels + 1
        for i, o in enumerate(outs):
            assert torch.equal(o, generic), f"thread {i}: max diff {float((o - generic).abs().max())}"
        # a later call finds the kernel in the cache
        again = sp.decode_attn(lay, q, dck, dcv, cap, ctx, ups["K"], ups["V"], scale)
        torch.cuda.synchronize()
        assert torch.equal(again, generic)
        assert sp.jit_kernel_count() == n_kernels + 1
        _flush(f"    {N_THREADS} concurrent first calls and one cached call: bit-identical to the generic kernel")
    finally:
        sp.set_jit(prev)
