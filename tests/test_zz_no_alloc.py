"""The no-allocation decode entry point (spectra_decode_attn_noalloc) through the C ABI: its
output equals spectra_decode_attn's bit for bit (the same kernels on the same inputs; only the
workspace differs), on two calls in a row, the second smaller than the first, so that the second
reads a scratch array that still holds the first call's partials."""
import ctypes
import math
import sys

import numpy as np
import pytest

from synth import generators as gen
import spectral_transform_coding_amd as sp
from tests import helpers as H
from tests.test_gpu_parity import SHAPES

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(name, ctx, cap, seed, with_wo=False):
    import torch
    d, hq, kv, dh, ns, r, g, wk, wv, dt = SHAPES[name]
    olay, lay = H.make_layouts(d, hq, kv, dh, ns, r, g, wk, wv)
    rng = np.random.default_rng(seed)
    B = len(ctx)
    ck, cv, _ = H.build_caches(olay, B, cap, ctx, rng, outlier_frac=0.01)
    ups = {}
    for kind in ("K", "V"):
        rows = [H.orthonormal_rows(olay.r_act_seg(kind, s), olay.seg_cols, rng) for s in range(olay.n_seg)]
        ups[kind] = H.to_dev(gen.input_dtype_round(np.concatenate(rows, axis=0), dt), dt)
    q = H.to_dev(gen.input_dtype_round(rng.standard_normal((B, hq, dh)), dt), dt)
    wo = H.to_dev(gen.input_dtype_round(rng.standard_normal((hq * dh, d)) / math.sqrt(hq * dh), dt), dt) if with_wo else None
    dck, dcv = H.dev_bytes(ck), H.dev_bytes(cv)
    scale = 1.0 / math.sqrt(dh)
    # the existing entry point, with its own workspace
    ref = sp.decode_attn(lay, q, dck, dcv, cap, ctx, ups["K"], ups["V"], scale, w_o=wo)
    # the new one, straight through the C ABI (no workspace argument)
    out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device="cuda")
    cl, clp = sp._i32(ctx, B, "ctx_len")
    st = sp.lib().spectra_decode_attn_noalloc(lay.c, sp._dtype_code(q), sp._ptr(q), sp._ptr(dck), sp._ptr(dcv),
                                              cap, B, clp, sp._ptr(ups["K"]), sp._ptr(ups["V"]), ctypes.c_float(scale),
                                              sp._ptr(wo), sp._ptr(out), sp._stream(None))
    assert st == sp.OK, sp.lib().spectra_last_error()
    torch.cuda.synchronize()
    a, b = ref.cpu().numpy(), out.cpu().numpy()
    assert np.isfinite(a).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), float(np.abs(a - b).max())
    _flush(f"    {name} ctx={ctx}: no-allocation output bit-identical")


@pytest.mark.parametrize("name", ["llama_4bit", "perhead_r6", "small_g4_bf16"])
def test_noalloc_matches_workspace_entry_point_two_calls(name):
    _flush(f"[noalloc] {name}")
    _case(name, [2000, 1500, 77, 1024], 2048, seed=41)      # larger first
    _case(name, [300, 129], 384, seed=42)                    # then smaller, over its leftovers


def test_noalloc_output_projection_and_empty_context():
    _flush("[noalloc] llama_4bit with W_O and an empty context")
    _case("llama_4bit", [0, 640, 33], 640, seed=43, with_wo=True)


@pytest.mark.parametrize("name", ["llama_4bit", "h40_bf16"])
def test_noalloc_every_key_group_split_two_calls(name):
    # The key-score split switch chooses the stream kernel's specialisation; the no-allocation
    # entry point must follow it exactly as the workspace entry point does.
    _flush(f"[noalloc] {name} with every key group split")
    prev = sp.set_key_split(1)
    try:
        _case(name, [2000, 1500, 77, 1024], 2048, seed=44)
        _case(name, [300, 129], 384, seed=45)
    finally:
        sp.set_key_split(prev)
