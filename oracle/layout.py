"""Packed latent-cache layout (oracle).

The pages fix no bit layout; they only require the cache to stay append-only, which is why
coordinates are grouped under one width ([SPECTRA] SPECTRA pipeline, stage 2, grouping).
This file states the layout this project uses, as a definition; the HIP library implements
the same definition independently.

One buffer per tensor (K or V).  Sequence b owns ceil(capacity / 128) consecutive blocks;
block n holds token positions 128 n .. 128 n + 127 ("slots" tau = 0..127).
A block is:  [code chunk of every (segment s, active group k), in order]
             [scale chunk of every (segment s, active group k), in the same order]
Code chunk of a group with width b: 128 * g codes, 16 g b bytes.  The code of (slot tau,
coordinate j) sits at position p = pos(kind, g, tau, j) and occupies bits [p b, p b + b) of
the chunk read as a little-endian bit stream (bit q is bit q & 7 of byte q >> 3).
Scale chunk: 128 fp16 values (256 bytes); the scale of slot tau is entry scale_index(tau):
  slot order (tau) except for K with g == 16, where entry 4 m + T holds the scale of slot
  32 T + t with m = 8 ((t >> 2) & 3) + 4 (t >> 4) + (t & 3) (the four scales a K run's
  tokens need are adjacent).

pos():
  g != 16:  p = tau * g + j                                     (token-major)
  g == 16:  p = 32 L + 8 T + e with tau = 32 T + t, and
     K:  j = 8 H + e,  m = 8 ((t >> 2) & 3) + 4 (t >> 4) + (t & 3),  L = 32 H + m
     V:  t = 8 q + e,  L = 16 q + j
  i.e. the chunk holds 64 runs ("lanes" L) of 32 codes, each run b whole 32-bit words.  For K a
  run holds 8 consecutive coordinates of one token in each of the block's four 32-token
  quarters; for V a run holds one coordinate of 8 consecutive tokens in each quarter.

Bits of a code (bit k of the code, k = 0..b-1):
  g != 16:  chunk bit p b + k (a plain little-endian bit stream).
  g == 16:  run L owns b 32-bit words; its word w (w = 0..b-1) is word 64 w + L of the chunk
            (word-major: the runs' first words, then their second words, ...).  The run's 32
            codes form 16 pairs i = 4 T + e // 2; the even-e code of a pair belongs to stream 0
            (the low 16 bits of each of the run's words), the odd-e code to stream 1 (the high
            16 bits).  Stream bit gamma = i b + k lives in run word gamma // 16 at bit
            16 * (e % 2) + gamma % 16, so
            chunk bit = 32 (64 (gamma // 16) + L) + 16 (e % 2) + gamma % 16.
  The two codes of a pair sit at the same offset in the two halves of a word, which is the
  order in which the decode kernel's matrix-core operands consume them (two fp16 values per
  32-bit register).  A lane L reads its b words, no code crosses into another lane's words,
  and word w of all 64 runs is one contiguous 256-byte row.
"""
import numpy as np

BT = 128          # tokens per block
SCALE_BYTES = 2   # fp16


def pos(kind: str, g: int, tau, j):
    """Code position of (slot tau, coordinate j) inside a group's code chunk."""
    tau = np.asarray(tau, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    if g != 16:
        return tau * g + j
    T, t = tau // 32, tau % 32
    if kind == "K":
        H, e = j // 8, j % 8
        m = 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3)
        L = 32 * H + m
    elif kind == "V":
        q, e = t // 8, t % 8
        L = 16 * q + j
    else:
        raise ValueError(kind)
    return 32 * L + 8 * T + e


def scale_index(kind: str, g: int, tau):
    """Entry of a scale chunk holding the scale of slot tau."""
    tau = np.asarray(tau, dtype=np.int64)
    if g != 16 or kind != "K":
        return tau
    T, t = tau // 32, tau % 32
    m = 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3)
    return 4 * m + T


def bit_loc(kind: str, g: int, b: int, tau, j, k):
    """Chunk bit holding bit k of the code of (slot tau, coordinate j), width b."""
    p = pos(kind, g, tau, j)
    k = np.asarray(k, dtype=np.int64)
    if g != 16:
        return p * b + k
    L, rest = p // 32, p % 32
    T, e = rest // 8, rest % 8
    i = 4 * T + e // 2
    gamma = i * b + k
    return 32 * (64 * (gamma // 16) + L) + 16 * (e % 2) + gamma % 16


class Layout:
    """Shapes of one layer's packed cache.  widths_k / widths_v: int [n_seg, seg_rank/g]."""

    def __init__(self, d_model, n_q_heads, n_kv_heads, d_head, n_seg, seg_rank, group_size,
                 widths_k, widths_v):
        self.d_model, self.n_q_heads, self.n_kv_heads, self.d_head = d_model, n_q_heads, n_kv_heads, d_head
        self.n_seg, self.seg_rank, self.g = n_seg, seg_rank, group_size
        assert n_kv_heads % n_seg == 0 and n_q_heads % n_kv_heads == 0
        assert seg_rank % group_size == 0
        self.n_groups = seg_rank // group_size
        self.widths = {
            "K": np.asarray(widths_k, dtype=np.int64).reshape(n_seg, self.n_groups),
            "V": np.asarray(widths_v, dtype=np.int64).reshape(n_seg, self.n_groups),
        }
        assert all(((w >= 0) & (w <= 8)).all() for w in self.widths.values())
        self.seg_cols = n_kv_heads * d_head // n_seg
        self.kv_per_seg = n_kv_heads // n_seg

    # --- groups and columns -------------------------------------------------------------
    def chunks(self, kind):
        """Active (segment, group, width) in storage order."""
        w = self.widths[kind]
        return [(s, k, int(w[s, k])) for s in range(self.n_seg) for k in range(self.n_groups)
                if w[s, k] > 0]

    def widths_active(self, kind):
        return [b for (_, _, b) in self.chunks(kind)]

    def r_act_seg(self, kind, s):
        return int(np.sum(self.widths[kind][s] > 0)) * self.g

    def r_act(self, kind):
        return sum(self.r_act_seg(kind, s) for s in range(self.n_seg))

    def seg_row_offset(self, kind, s):
        return sum(self.r_act_seg(kind, t) for t in range(s))

    def kv_head(self, h):
        return h // (self.n_q_heads // self.n_kv_heads)

    # --- bytes ----------------------------------------------------------------------------
    def code_chunk_bytes(self, b):
        return BT * self.g * b // 8

    def block_bytes(self, kind):
        return sum(self.code_chunk_bytes(b) + BT * SCALE_BYTES for (_, _, b) in self.chunks(kind))

    def offsets(self, kind):
        """(code offsets, scale offsets) of the active chunks inside a block."""
        ch = self.chunks(kind)
        code_off, o = [], 0
        for (_, _, b) in ch:
            code_off.append(o)
            o += self.code_chunk_bytes(b)
        scale_off = [o + i * BT * SCALE_BYTES for i in range(len(ch))]
        return code_off, scale_off

    def n_blocks(self, cap_tokens):
        return (int(cap_tokens) + BT - 1) // BT

    def empty_cache(self, kind, batch, cap_tokens):
        return np.zeros((batch, self.n_blocks(cap_tokens), self.block_bytes(kind)), dtype=np.uint8)

    def bits_per_token(self, kind):
        return sum(self.g * b + 16 for (_, _, b) in self.chunks(kind))


def write_tokens(lay: Layout, kind: str, cache: np.ndarray, b: int, positions, u, s16):
    """OR the codes u [n, r_act] and store the scales s16 [n, n_active] of tokens at the
    given cache positions of sequence b.  Bits of other tokens are left as they are."""
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size == 0:
        return
    u = np.asarray(u, dtype=np.uint8)
    s16 = np.asarray(s16, dtype=np.float16)
    blk, tau = positions // BT, positions % BT
    code_off, scale_off = lay.offsets(kind)
    g = lay.g
    ublk = np.unique(blk)
    bmap = {int(x): i for i, x in enumerate(ublk)}
    bi = np.array([bmap[int(x)] for x in blk])
    for ci, (_, _, bw) in enumerate(lay.chunks(kind)):
        nbits = BT * g * bw
        bits = np.zeros((ublk.size, nbits), dtype=np.uint8)
        j = np.arange(g)
        codes = u[:, ci * g:(ci + 1) * g].astype(np.int64)              # [n, g]
        for i in range(bw):
            bits[bi[:, None], bit_loc(kind, g, bw, tau[:, None], j[None, :], i)] = (codes >> i) & 1
        packed = np.packbits(bits, axis=1, bitorder="little")           # [nb, nbits/8]
        lo = code_off[ci]
        cache[b, ublk, lo:lo + nbits // 8] |= packed
        sb = np.ascontiguousarray(s16[:, ci]).view(np.uint8).reshape(-1, 2)
        so = scale_off[ci] + 2 * scale_index(kind, g, tau)
        cache[b, blk, so] = sb[:, 0]
        cache[b, blk, so + 1] = sb[:, 1]


def read_tokens(lay: Layout, kind: str, cache: np.ndarray, b: int, positions):
    """Codes [n, r_act] uint8 and scales [n, n_active] float16 of the given positions."""
    positions = np.asarray(positions, dtype=np.int64)
    n = positions.size
    blk, tau = positions // BT, positions % BT
    code_off, scale_off = lay.offsets(kind)
    g = lay.g
    ch = lay.chunks(kind)
    u = np.zeros((n, len(ch) * g), dtype=np.uint8)
    s = np.zeros((n, len(ch)), dtype=np.float16)
    j = np.arange(g)
    for ci, (_, _, bw) in enumerate(ch):
        val = np.zeros((n, g), dtype=np.int64)
        for i in range(bw):
            q = bit_loc(kind, g, bw, tau[:, None], j[None, :], i)
            byte = cache[b, blk[:, None], code_off[ci] + (q >> 3)].astype(np.int64)
            val |= ((byte >> (q & 7)) & 1) << i
        u[:, ci * g:(ci + 1) * g] = val.astype(np.uint8)
        so = scale_off[ci] + 2 * scale_index(kind, g, tau)
        pair = np.stack([cache[b, blk, so], cache[b, blk, so + 1]], axis=1).copy()
        s[:, ci] = pair.view(np.float16)[:, 0]
    return u, s
