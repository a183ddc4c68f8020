"""The no-allocation decode entry point captured into a HIP graph (torch.cuda.CUDAGraph): the
library allocates nothing and clears nothing with memsets inside the call, so the captured launches
replay as they ran. Each replay, with eager work and synchronisations between replays, must equal
the eager call bit for bit, and a replay after the query buffer is overwritten in place must equal
an eager call on the new query (the graph reads its input buffers at replay time)."""
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


@pytest.mark.parametrize("name", ["llama_4bit", "perhead_r6"])
def test_noalloc_decode_graph_replays_match_eager(name):
    import torch
    _flush(f"[graph] {name}: no-allocation decode captured and replayed")
    d, hq, kv, dh, ns, r, g, wk, wv, dt = SHAPES[name]
    olay, lay = H.make_layouts(d, hq, kv, dh, ns, r, g, wk, wv)
    rng = np.random.default_rng(81)
    ctx, cap = [1500, 640, 77, 1024], 1536
    B = len(ctx)
    ck, cv, _ = H.build_caches(olay, B, cap, ctx, rng, outlier_frac=0.01)
    ups = {}
    for kind in ("K", "V"):
        rows = [H.orthonormal_rows(olay.r_act_seg(kind, s), olay.seg_cols, rng) for s in range(olay.n_seg)]
        ups[kind] = H.to_dev(gen.input_dtype_round(np.concatenate(rows, axis=0), dt), dt)
    q = H.to_dev(gen.input_dtype_round(rng.standard_normal((B, hq, dh)), dt), dt)
    q2 = H.to_dev(gen.input_dtype_round(rng.standard_normal((B, hq, dh)), dt), dt)
    dck, dcv = H.dev_bytes(ck), H.dev_bytes(cv)
    scale = 1.0 / math.sqrt(dh)

    def eager(qq):
        o = sp.decode_attn(lay, qq, dck, dcv, cap, ctx, ups["K"], ups["V"], scale)
        torch.cuda.synchronize()
        return o

    ref, ref2 = eager(q), eager(q2)          # the first call also builds any specialised kernel
    assert np.isfinite(ref.cpu().numpy()).all() and not torch.equal(ref, ref2)
    qin = q.clone()
    out = torch.full_like(ref, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm-up on a side stream before the capture
        sp.decode_attn_noalloc(lay, qin, dck, dcv, cap, ctx, ups["K"], ups["V"], scale, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sp.decode_attn_noalloc(lay, qin, dck, dcv, cap, ctx, ups["K"], ups["V"], scale, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}: max diff {float((out - ref).abs().max())}"
        assert torch.equal(eager(q2), ref2)   # eager work between replays
    qin.copy_(q2)
    out.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)
    del graph
    _flush(f"    {name}: 5 replays bit-identical to eager calls")
