"""Reconstruct-then-attend decode and the encode path (oracle, float64).

[SPECTRA] SPECTRA pipeline, stage 3: at inference the full keys and values are rebuilt on the
fly from the latent cache and used in standard attention; the latent is appended per token
after down-projection and per-token quantisation.  This oracle follows that literal order:
unpack -> dequantise -> K^ = C^ W_up, V^ = C^ W_up per key/value head -> softmax attention.
(The GPU computes the same result in latent space; the pages name latent-space attention as
the route to saving compute, [SPECTRA] Significance.)

Readings: softmax scale is given by the caller (1/sqrt(d_head) in the workloads); query head h
uses key/value head h // (n_q_heads / n_kv_heads); no positional rotation (the pages fold
W_down into fixed weights, which a rotation would break); a query attends to the first
ctx_len[b] cached tokens, including the one just appended.
"""
import numpy as np

from . import layout as L
from . import quant


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Standard attention for one query vector: softmax(scale K q) V, max-subtracted, fp64."""
    s = (np.asarray(K, np.float64) @ np.asarray(q, np.float64)) * scale
    s = s - s.max()
    p = np.exp(s)
    return (p / p.sum()) @ np.asarray(V, np.float64)


def reconstruct(lay: L.Layout, kind: str, chat: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """Full keys or values [T, n_kv * d_head] from dequantised latent rows chat [T, r_act].
    w_up [r_act, seg_cols] holds each segment's rows in order."""
    T = chat.shape[0]
    out = np.zeros((T, lay.n_kv_heads * lay.d_head), dtype=np.float64)
    w_up = np.asarray(w_up, dtype=np.float64)
    for s in range(lay.n_seg):
        r0, r = lay.seg_row_offset(kind, s), lay.r_act_seg(kind, s)
        cols = slice(s * lay.seg_cols, (s + 1) * lay.seg_cols)
        out[:, cols] = chat[:, r0:r0 + r] @ w_up[r0:r0 + r, :]
    return out


def attend_all_heads(lay: L.Layout, q_b: np.ndarray, Kf: np.ndarray, Vf: np.ndarray,
                     scale: float) -> np.ndarray:
    """o [Hq, d_head] for one sequence from full keys/values [T, n_kv*d_head]."""
    dh = lay.d_head
    o = np.zeros((lay.n_q_heads, dh), dtype=np.float64)
    for h in range(lay.n_q_heads):
        kv = lay.kv_head(h)
        o[h] = softmax_attention(q_b[h], Kf[:, kv * dh:(kv + 1) * dh], Vf[:, kv * dh:(kv + 1) * dh], scale)
    return o


def dequantized_latents(lay: L.Layout, kind: str, cache: np.ndarray, b: int, ctx: int):
    u, s = L.read_tokens(lay, kind, cache, b, np.arange(ctx))
    return quant.dequantize_latent(u, s, lay.widths_active(kind), lay.g)


def decode(lay: L.Layout, q: np.ndarray, cache_k: np.ndarray, cache_v: np.ndarray, ctx_len,
           w_up_k: np.ndarray, w_up_v: np.ndarray, scale: float, w_o: np.ndarray = None,
           heads=None):
    """Decode attention over the packed caches.  q [B, Hq, d_head].
    Returns o [B, Hq, d_head] (float64), or y = concat_h(o_h) W_O [B, d_model] if w_o is
    given.  `heads`, if given, restricts the computation to those (b, h) pairs (others 0)."""
    B = q.shape[0]
    o = np.zeros((B, lay.n_q_heads, lay.d_head), dtype=np.float64)
    for b in range(B):
        want = None if heads is None else [h for (bb, h) in heads if bb == b]
        if want is not None and not want:
            continue
        ctx = int(ctx_len[b])
        if ctx == 0:
            continue
        Kf = reconstruct(lay, "K", dequantized_latents(lay, "K", cache_k, b, ctx), w_up_k)
        Vf = reconstruct(lay, "V", dequantized_latents(lay, "V", cache_v, b, ctx), w_up_v)
        dh = lay.d_head
        for h in (range(lay.n_q_heads) if want is None else want):
            kv = lay.kv_head(h)
            o[b, h] = softmax_attention(q[b, h], Kf[:, kv * dh:(kv + 1) * dh],
                                        Vf[:, kv * dh:(kv + 1) * dh], scale)
    if w_o is None:
        return o
    return o.reshape(B, -1) @ np.asarray(w_o, dtype=np.float64)


def encode_latent(x: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """Latent rows c = x W_down in float64 (W_down [d_model, r_act_k + r_act_v])."""
    return np.asarray(x, np.float64) @ np.asarray(w_down, np.float64)


def append(lay: L.Layout, cache_k, cache_v, latent32: np.ndarray, batch: int, n_new: int,
           start_pos):
    """Quantise float32 latent rows [batch * n_new, r_act_k + r_act_v] (row b * n_new + i is
    token i of sequence b) and write them at positions start_pos[b] + i."""
    rk = lay.r_act("K")
    lat = np.asarray(latent32, dtype=np.float32).reshape(batch, n_new, -1)
    for kind, cache, cols in (("K", cache_k, slice(0, rk)), ("V", cache_v, slice(rk, None))):
        for b in range(batch):
            u, s = quant.quantize_latent(lat[b, :, cols], lay.widths_active(kind), lay.g)
            L.write_tokens(lay, kind, cache, b, int(start_pos[b]) + np.arange(n_new), u, s)
