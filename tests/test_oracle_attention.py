"""Pins for oracle.attention: reconstruct-then-attend decode (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attention as A, layout as L, quant, transform, calibrate


def _brute_attention(q, K, V, scale):
    """Pure-Python loops: scores, max, exp, normalise, weighted sum."""
    T, dh = len(K), len(V[0])
    sc = [scale * sum(q[i] * K[t][i] for i in range(len(q))) for t in range(T)]
    m = max(sc)
    e = [math.exp(x - m) for x in sc]
    z = sum(e)
    return [sum(e[t] * V[t][d] for t in range(T)) / z for d in range(dh)]


def _setup(d=32, n_kv=2, dh=8, Hq=4, T=40, seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((500, d)) @ np.diag(np.arange(1, d + 1) ** -0.7)
    G = transform.gram(X)
    wk = rng.standard_normal((d, n_kv * dh)) / math.sqrt(d)
    wv = rng.standard_normal((d, n_kv * dh)) / math.sqrt(d)
    h = rng.standard_normal((T, d)) @ np.diag(np.arange(1, d + 1) ** -0.7)
    q = rng.standard_normal((1, Hq, dh))
    return G, wk, wv, h, q


def _exact_decode(lay, G, wk, wv, h, q, r, scale):
    """Decode from the unquantised latent through the oracle's reconstruct + attend."""
    lk, Vk = transform.g_weighted_eig(G, wk)
    lv, Vv = transform.g_weighted_eig(G, wv)
    ck, cv = h @ wk @ Vk[:, :r], h @ wv @ Vv[:, :r]
    Kf = A.reconstruct(lay, "K", ck, Vk[:, :r].T)
    Vf = A.reconstruct(lay, "V", cv, Vv[:, :r].T)
    return A.attend_all_heads(lay, q[0], Kf, Vf, scale), Vk, Vv


def test_full_rank_without_quantisation_is_exact_attention():
    # (3): full rank, no quantisation -> standard attention on K = h W_K, V = h W_V
    G, wk, wv, h, q = _setup()
    n_kv, dh, Hq = 2, 8, 4
    lay = L.Layout(32, Hq, n_kv, dh, 1, 16, 4, np.full((1, 4), 8), np.full((1, 4), 8))
    o, _, _ = _exact_decode(lay, G, wk, wv, h, q, 16, 1 / math.sqrt(dh))
    K, V = h @ wk, h @ wv
    for hh in range(Hq):
        kv = hh // (Hq // n_kv)
        ref = _brute_attention(q[0, hh].tolist(), K[:, kv * dh:(kv + 1) * dh].tolist(),
                               V[:, kv * dh:(kv + 1) * dh].tolist(), 1 / math.sqrt(dh))
        assert np.allclose(o[hh], ref, rtol=1e-11, atol=1e-12)


def test_zero_bit_tail_is_rank_r_truncated_attention():
    # (4): tail groups at 0 bits, head groups unquantised -> attention on rank-r projected keys
    G, wk, wv, h, q = _setup(seed=1)
    n_kv, dh, Hq, r = 2, 8, 4, 8
    lay = L.Layout(32, Hq, n_kv, dh, 1, 16, 4, np.array([[8, 8, 0, 0]]), np.array([[8, 8, 0, 0]]))
    assert lay.r_act("K") == r
    o, Vk, Vv = _exact_decode(lay, G, wk, wv, h, q, r, 1 / math.sqrt(dh))
    Kr = h @ wk @ Vk[:, :r] @ Vk[:, :r].T
    Vr = h @ wv @ Vv[:, :r] @ Vv[:, :r].T
    for hh in range(Hq):
        kv = hh // (Hq // n_kv)
        ref = _brute_attention(q[0, hh].tolist(), Kr[:, kv * dh:(kv + 1) * dh].tolist(),
                               Vr[:, kv * dh:(kv + 1) * dh].tolist(), 1 / math.sqrt(dh))
        assert np.allclose(o[hh], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("T", [1, 2, 5])
def test_packed_decode_matches_brute_force_on_tiny_heads(T):
    # (5): tiny heads (d = 8, d_h = 4), packed cache, loops vs the vectorised oracle
    rng = np.random.default_rng(T)
    d, n_kv, dh, Hq = 8, 2, 4, 4
    X = rng.standard_normal((64, d))
    G = transform.gram(X)
    wk = rng.standard_normal((d, n_kv * dh))
    wv = rng.standard_normal((d, n_kv * dh))
    cal = calibrate.calibrate(G, wk, wv, 1, 8, 2, 3.0)
    lay = L.Layout(d, Hq, n_kv, dh, 1, 8, 2, cal["k"]["widths"], cal["v"]["widths"])
    h = rng.standard_normal((T, d))
    lat = (h @ cal["w_down"]).astype(np.float32)
    ck, cv = lay.empty_cache("K", 1, T), lay.empty_cache("V", 1, T)
    A.append(lay, ck, cv, lat, 1, T, [0])
    q = rng.standard_normal((1, Hq, dh))
    scale = 1 / math.sqrt(dh)
    o = A.decode(lay, q, ck, cv, [T], cal["k"]["w_up"], cal["v"]["w_up"], scale)
    # brute force: dequantise code by code, rebuild keys/values coordinate by coordinate
    rk = lay.r_act("K")
    for hh in range(Hq):
        kv = hh // 2
        Ks, Vs = [], []
        for t in range(T):
            krow, vrow = [], []
            for kind, out, up, off in (("K", krow, cal["k"]["w_up"], 0), ("V", vrow, cal["v"]["w_up"], rk)):
                ws = lay.widths_active(kind)
                chat = []
                for gi, b in enumerate(ws):
                    grp = lat[t, off + 2 * gi: off + 2 * gi + 2]
                    u, s = quant.quantize(grp[None, :], b)
                    chat += [float(s[0]) * (int(x) - (2 ** b - 1) / 2) for x in u[0]]
                for c in range(kv * dh, (kv + 1) * dh):
                    out.append(sum(chat[i] * up[i, c] for i in range(len(chat))))
            Ks.append(krow)
            Vs.append(vrow)
        ref = _brute_attention(q[0, hh].tolist(), Ks, Vs, scale)
        assert np.allclose(o[0, hh], ref, rtol=1e-10, atol=1e-12)


def test_single_token_identical_keys_and_shift_invariance():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((6, 3))
    q = rng.standard_normal(4)
    K1 = rng.standard_normal((1, 4))
    assert np.allclose(A.softmax_attention(q, K1, V[:1], 0.5), V[0])
    Ksame = np.repeat(rng.standard_normal((1, 4)), 6, axis=0)
    assert np.allclose(A.softmax_attention(q, Ksame, V, 0.5), V.mean(axis=0))
    K = rng.standard_normal((6, 4))
    # adding a constant to every score (a key offset along q) leaves the output unchanged
    shift = 3.0 * q / np.dot(q, q)
    assert np.allclose(A.softmax_attention(q, K, V, 1.0), A.softmax_attention(q, K + shift, V, 1.0))


def test_gqa_head_mapping_and_output_projection():
    lay = L.Layout(64, 8, 2, 4, 1, 8, 4, np.array([[8, 8]]), np.array([[8, 8]]))
    assert [lay.kv_head(h) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    rng = np.random.default_rng(5)
    up = np.linalg.qr(rng.standard_normal((8, 8)))[0]
    ck, cv = lay.empty_cache("K", 2, 10), lay.empty_cache("V", 2, 10)
    lat = rng.standard_normal((20, 16)).astype(np.float32)
    A.append(lay, ck, cv, lat, 2, 10, [0, 0])
    q = rng.standard_normal((2, 8, 4))
    wo = rng.standard_normal((32, 64))
    o = A.decode(lay, q, ck, cv, [10, 7], up, up, 0.5)
    y = A.decode(lay, q, ck, cv, [10, 7], up, up, 0.5, w_o=wo)
    assert np.allclose(y, o.reshape(2, 32) @ wo)
    # ctx_len limits what is read: the shorter sequence ignores its tail
    o7 = A.decode(lay, q[1:], ck[1:], cv[1:], [7], up, up, 0.5)
    assert np.allclose(o7[0], o[1])


def test_per_head_segments_reconstruct_their_own_head():
    # with one segment per KV head, W_up rows of segment s only touch head s's columns
    lay = L.Layout(16, 4, 2, 4, 2, 4, 2, np.array([[4, 4], [4, 0]]), np.array([[4, 4], [4, 4]]))
    assert lay.r_act("K") == 6 and lay.seg_row_offset("K", 1) == 4
    up = np.arange(6 * 4, dtype=float).reshape(6, 4)
    chat = np.ones((1, 6))
    full = A.reconstruct(lay, "K", chat, up)
    assert np.allclose(full[0, :4], up[:4].sum(axis=0))
    assert np.allclose(full[0, 4:], up[4:].sum(axis=0))
