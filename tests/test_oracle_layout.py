"""Pins for oracle.layout: the packed cache layout (CPU only)."""
import os

import numpy as np
import pytest

from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lay(g, wk, wv=None, n_seg=1, rank=None, kv=1, dh=None):
    wk = np.asarray(wk)
    wv = wk if wv is None else np.asarray(wv)
    rank = rank or wk.shape[-1] * g
    dh = dh or 64
    return L.Layout(256, kv, kv, dh, n_seg, rank, g, wk, wv)


def test_hand_computed_block():
    lay = _lay(2, [[3, 1]], rank=4)
    assert lay.block_bytes("K") == 640
    cache = lay.empty_cache("K", 1, 128)
    u = np.array([[5, 2, 1, 0], [7, 1, 0, 1]], dtype=np.uint8)
    s = np.array([[1.0, 2.0], [0.5, 0.25]], dtype=np.float16)
    L.write_tokens(lay, "K", cache, 0, [0, 1], u, s)
    expect = np.zeros(640, dtype=np.uint8)
    for line in open(os.path.join(GOLDEN, "pack_g2_w31.txt")):
        if line.startswith("#") or not line.strip():
            continue
        off, val = line.split()
        expect[int(off)] = int(val, 16)
    assert np.array_equal(cache[0, 0], expect)


def test_hand_computed_g16_positions():
    # K, slot 5 (quarter 0, t = 5), width 8, code of coordinate j = j + 1:
    #   coords 0..7 -> run m = 8*((5>>2)&3) + 4*(5>>4) + (5&3) = 9;
    #   coordinate e -> pair i = e//2, stream e%2, stream bit 8i -> run word i//2, bit 16(e%2) + 8(i%2)
    #   -> chunk word 64(i//2) + 9, byte 4(64(i//2) + 9) + 2(e%2) + (i%2):
    #   codes 1..4 land in bytes 36..39 as 1,3,2,4 and codes 5..8 in bytes 292..295 as 5,7,6,8.
    #   coords 8..15 -> run 41: words 41 and 105 (bytes 164.. and 420..), same order.
    # V, slot 5: quarter 0, q = 0, e = 5 -> run j, pair i = 2, stream 1 -> run word 1, bit 16
    #   -> chunk word 64 + j, byte 4(64 + j) + 2 = 258 + 4 j.
    lay = _lay(16, [[8]], rank=16)
    u = np.arange(1, 17, dtype=np.uint8)[None, :]
    s = np.array([[1.0]], dtype=np.float16)
    ck = lay.empty_cache("K", 1, 128)
    L.write_tokens(lay, "K", ck, 0, [5], u, s)
    assert ck[0, 0, 36:40].tolist() == [1, 3, 2, 4]
    assert ck[0, 0, 292:296].tolist() == [5, 7, 6, 8]
    assert ck[0, 0, 164:168].tolist() == [9, 11, 10, 12]
    assert ck[0, 0, 420:424].tolist() == [13, 15, 14, 16]
    assert int(np.count_nonzero(ck[0, 0, :2048])) == 16
    # K scale of slot 5 (m = 9, T = 0) is entry 4*9 + 0 = 36 of the scale chunk: fp16 1.0
    assert ck[0, 0, 2048 + 72:2048 + 74].tolist() == [0x00, 0x3C]
    assert int(np.count_nonzero(ck[0, 0, 2048:])) == 1
    cv = lay.empty_cache("V", 1, 128)
    L.write_tokens(lay, "V", cv, 0, [5], u, s)
    assert [int(cv[0, 0, 258 + 4 * j]) for j in range(16)] == list(range(1, 17))
    assert int(np.count_nonzero(cv[0, 0, :2048])) == 16
    # V scales stay in slot order: entry 5
    assert cv[0, 0, 2048 + 10:2048 + 12].tolist() == [0x00, 0x3C]


def test_hand_computed_g16_straddling_code():
    # width 3, K: slot 32 is quarter T = 1, t = 0 -> run m = 0; its coordinates 0..7 form
    # pairs 4..7 at stream bits 12..23, so pair 5 (stream bits 15..17) straddles run words 0
    # and 1, i.e. chunk words 0 and 64.
    lay = _lay(16, [[3]], rank=16)
    u = np.zeros((1, 16), dtype=np.uint8)
    u[0, 2] = 7        # coordinate 2 of slot 32: quarter 1, e = 2 -> pair 5, stream 0
    s = np.array([[1.0]], dtype=np.float16)
    ck = lay.empty_cache("K", 1, 128)
    L.write_tokens(lay, "K", ck, 0, [32], u, s)
    # gamma = 15, 16, 17 -> chunk word 0 bit 15, chunk word 64 bits 0 and 1
    # -> byte 1 = 0x80, byte 256 = 0x03
    nz = {int(i): int(ck[0, 0, i]) for i in np.nonzero(ck[0, 0, :768])[0]}   # code bytes only
    assert nz == {1: 0x80, 256: 0x03}
    # scale of slot 32 (T = 1, m = 0): entry 1
    assert ck[0, 0, 768 + 2:768 + 4].tolist() == [0x00, 0x3C]


@pytest.mark.parametrize("g", [2, 4, 16])
@pytest.mark.parametrize("kind", ["K", "V"])
def test_pos_is_a_bijection(g, kind):
    tau, j = np.meshgrid(np.arange(128), np.arange(g), indexing="ij")
    p = L.pos(kind, g, tau, j).ravel()
    assert np.array_equal(np.sort(p), np.arange(128 * g))


@pytest.mark.parametrize("kind", ["K", "V"])
def test_g16_lane_runs(kind):
    # bit locations of every code stay inside its run's b words (chunk words 64 w + L)
    for b in range(1, 9):
        tau, j = np.meshgrid(np.arange(128), np.arange(16), indexing="ij")
        p = L.pos(kind, 16, tau, j)
        for k in range(b):
            word = L.bit_loc(kind, 16, b, tau, j, k) // 32
            assert np.all(word % 64 == p // 32) and np.all(word // 64 < b)
        allbits = np.stack([L.bit_loc(kind, 16, b, tau, j, k) for k in range(b)]).ravel()
        assert np.array_equal(np.sort(allbits), np.arange(128 * 16 * b))

    # each run of 32 positions (one lane) holds, per 32-token quarter T, 8 codes that are
    # consecutive coordinates of one token (K) or one coordinate of 8 consecutive tokens (V)
    tau, j = np.meshgrid(np.arange(128), np.arange(16), indexing="ij")
    p = L.pos(kind, 16, tau, j)
    inv = {}
    for t in range(128):
        for c in range(16):
            inv[int(p[t, c])] = (t, c)
    for lane in range(64):
        for T in range(4):
            run = [inv[32 * lane + 8 * T + e] for e in range(8)]
            toks = [r[0] for r in run]
            coords = [r[1] for r in run]
            assert all(32 * T <= t < 32 * T + 32 for t in toks)
            if kind == "K":
                assert len(set(toks)) == 1 and coords == list(range(coords[0], coords[0] + 8))
            else:
                assert len(set(coords)) == 1 and toks == list(range(toks[0], toks[0] + 8))


@pytest.mark.parametrize("g", [2, 4, 16])
def test_round_trip_and_bits_per_token(g):
    rng = np.random.default_rng(g)
    G = 48 // g
    wk = rng.integers(0, 9, (2, G))
    wk[0, 0] = 8
    wv = rng.integers(0, 9, (2, G))
    wv[1, 0] = 1
    lay = L.Layout(256, 4, 2, 24, 2, 48, g, wk, wv)
    for kind in ("K", "V"):
        ws = lay.widths_active(kind)
        assert lay.bits_per_token(kind) == sum(g * b + 16 for b in ws)
        assert lay.block_bytes(kind) * 8 == 128 * lay.bits_per_token(kind)
        cache = lay.empty_cache(kind, 2, 300)
        pos = np.array([0, 1, 2, 127, 128, 129, 250, 299])
        u = np.zeros((pos.size, lay.r_act(kind)), dtype=np.uint8)
        for i, b in enumerate(ws):
            u[:, i * g:(i + 1) * g] = rng.integers(0, 2 ** b, (pos.size, g))
        s = rng.lognormal(0, 1, (pos.size, len(ws))).astype(np.float16)
        L.write_tokens(lay, kind, cache, 1, pos, u, s)
        assert np.all(cache[0] == 0)
        u2, s2 = L.read_tokens(lay, kind, cache, 1, pos)
        assert np.array_equal(u, u2) and np.array_equal(s, s2)


@pytest.mark.parametrize("g", [4, 16])
def test_append_one_token_changes_only_its_bits(g):
    rng = np.random.default_rng(21)
    G = 32 // g
    w = np.array([[7, 5, 3, 1, 2, 6, 4, 8][:G]])
    lay = L.Layout(128, 2, 1, 32, 1, 32, g, w, w)
    for kind in ("K", "V"):
        ws = lay.widths_active(kind)
        cache = lay.empty_cache(kind, 1, 256)
        pos = np.arange(0, 140)
        u = np.zeros((pos.size, lay.r_act(kind)), dtype=np.uint8)
        for i, b in enumerate(ws):
            u[:, i * g:(i + 1) * g] = rng.integers(0, 2 ** b, (pos.size, g))
        s = rng.lognormal(0, 1, (pos.size, len(ws))).astype(np.float16)
        L.write_tokens(lay, kind, cache, 0, pos[:-1], u[:-1], s[:-1])
        before = cache.copy()
        L.write_tokens(lay, kind, cache, 0, pos[-1:], u[-1:], s[-1:])
        changed = np.argwhere(cache != before)
        assert changed.size > 0 and np.all(changed[:, 1] == pos[-1] // 128)
        u2, s2 = L.read_tokens(lay, kind, cache, 0, pos)
        assert np.array_equal(u2, u) and np.array_equal(s2, s)
        # the new token's bits land only where its own codes live
        fresh = lay.empty_cache(kind, 1, 256)
        L.write_tokens(lay, kind, fresh, 0, pos[-1:], u[-1:], s[-1:])
        assert np.array_equal(cache ^ before, fresh)


def test_cache_geometry():
    lay = _lay(16, [[8, 7, 6]], rank=48)
    assert lay.n_blocks(1) == 1 and lay.n_blocks(128) == 1 and lay.n_blocks(129) == 2
    co, so = lay.offsets("K")
    assert co == [0, 2048, 2048 + 1792]
    assert so == [2048 + 1792 + 1536, 2048 + 1792 + 1536 + 256, 2048 + 1792 + 1536 + 512]
    assert all(o % 16 == 0 for o in co + so)


@pytest.mark.parametrize("b,tau,j,u,expect", [
    # V, g = 16: slot tau = 32 T + 8 q + e, run L = 16 q + j, pair i = 4 T + e // 2 in stream e % 2,
    # stream bits gamma = i b .. i b + b - 1; gamma < 16 in run word 0 (chunk word L), the rest in
    # run word 1 (chunk word 64 + L), at bit 16 (e % 2) + gamma % 16.  Each case straddles.
    # b = 3: tau 34 (T 1, q 0, e 2), j 5 -> L 5, pair 5, stream 0, gamma 15..17; u = 0b101:
    #   gamma 15 -> word 5 bit 15 (byte 21 = 0x80), gamma 17 -> word 69 bit 1 (byte 276 = 0x02)
    (3, 34, 5, 0b101, {21: 0x80, 276: 0x02}),
    # b = 5: tau 31 (T 0, q 3, e 7), j 9 -> L 57, pair 3, stream 1, gamma 15..19; u = 0b11001:
    #   gamma 15 (1) -> word 57 bit 31 (byte 231 = 0x80); gamma 16..19 (0, 0, 1, 1) -> word 121
    #   bits 16..19 -> bits 18, 19 (byte 486 = 0x0C)
    (5, 31, 9, 0b11001, {231: 0x80, 486: 0x0C}),
    # b = 6: tau 12 (T 0, q 1, e 4), j 0 -> L 16, pair 2, stream 0, gamma 12..17; u = 0b110011:
    #   gamma 12, 13 -> word 16 bits 12, 13 (byte 65 = 0x30); gamma 16, 17 -> word 80 bits 0, 1
    #   (byte 320 = 0x03)
    (6, 12, 0, 0b110011, {65: 0x30, 320: 0x03}),
    # b = 7: tau 21 (T 0, q 2, e 5), j 15 -> L 47, pair 2, stream 1, gamma 14..20; u = 0b1100101:
    #   gamma 14 (1) -> word 47 bit 30 (byte 191 = 0x40); gamma 16..20 (1, 0, 0, 1, 1) -> word 111
    #   bits 16, 19, 20 (byte 446 = 0x19)
    (7, 21, 15, 0b1100101, {191: 0x40, 446: 0x19}),
])
def test_hand_computed_g16_value_straddling_codes(b, tau, j, u, expect):
    lay = _lay(16, [[b]], rank=16)
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, j] = u
    s = np.array([[1.0]], dtype=np.float16)
    cv = lay.empty_cache("V", 1, 128)
    L.write_tokens(lay, "V", cv, 0, [tau], codes, s)
    cb = 16 * 16 * b
    nz = {int(i): int(cv[0, 0, i]) for i in np.nonzero(cv[0, 0, :cb])[0]}
    assert nz == expect
    # V scales in slot order: entry tau of the scale chunk after the codes holds fp16 1.0
    assert cv[0, 0, cb + 2 * tau:cb + 2 * tau + 2].tolist() == [0x00, 0x3C]
    assert int(np.count_nonzero(cv[0, 0, cb:])) == 1
    got_u, got_s = L.read_tokens(lay, "V", cv, 0, np.array([tau]))
    assert got_u[0].tolist() == codes[0].tolist()
