"""Python binding of libspectra (ctypes).  Argument marshalling only: every step of the codec
runs in the library (host calibration in C++, encode and decode in HIP kernels for gfx950).

The library must be built (`python spectral_transform_coding_amd/csrc/build.py`, or
`__graft_entry__.build()`); there is no fallback implementation.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspectra.so")

OK, EINVAL, ENOTSUP, ECAPACITY, EHIP, ENUMERIC = range(6)
F32, BF16 = 0, 1
TENSOR_K, TENSOR_V = 0, 1
BLOCK_TOKENS = 128
MAX_BATCH = 256

_STATUS = {0: "OK", 1: "EINVAL", 2: "ENOTSUP", 3: "ECAPACITY", 4: "EHIP", 5: "ENUMERIC"}


class SpectraError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("n_seg", ctypes.c_int32), ("seg_rank", ctypes.c_int32),
                ("group_size", ctypes.c_int32),
                ("widths_k", ctypes.POINTER(ctypes.c_uint8)),
                ("widths_v", ctypes.POINTER(ctypes.c_uint8))]


class _CalibParams(ctypes.Structure):
    _fields_ = [("n_seg", ctypes.c_int32), ("seg_rank", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("budget_bits", ctypes.c_double),
                ("fixed_width", ctypes.c_int32), ("energy", ctypes.c_double),
                ("scale_bits", ctypes.c_int32), ("max_width", ctypes.c_int32),
                ("rank_rule", ctypes.c_int32), ("gap_ratio", ctypes.c_double),
                ("rows", ctypes.POINTER(ctypes.c_double)), ("n_rows", ctypes.c_int64),
                ("robust", ctypes.c_int32), ("value_correction", ctypes.c_int32)]


_PD = ctypes.POINTER(ctypes.c_double)
_PU8 = ctypes.POINTER(ctypes.c_uint8)
_PI32 = ctypes.POINTER(ctypes.c_int32)


class _CalibOut(ctypes.Structure):
    _fields_ = [("w_down_t_k", _PD), ("w_down_t_v", _PD), ("w_up_k", _PD), ("w_up_v", _PD),
                ("widths_k", _PU8), ("widths_v", _PU8), ("sigma2_k", _PD), ("sigma2_v", _PD),
                ("theta_k", _PD), ("theta_v", _PD), ("energy_rank_k", _PI32),
                ("energy_rank_v", _PI32), ("r_act_k", ctypes.c_int32), ("r_act_v", ctypes.c_int32)]


SYMBOLS = ("spectra_calibrate", "spectra_cache_bytes", "spectra_block_bytes",
           "spectra_decode_workspace_bytes", "spectra_encode_append", "spectra_decode_attn",
           "spectra_unpack_dequant", "spectra_set_timing_events", "spectra_last_error",
           "spectra_version", "spectra_set_jit", "spectra_set_key_split", "spectra_jit_kernel_count",
           "spectra_decode_literal_workspace_bytes", "spectra_decode_attn_literal",
           "spectra_decode_attn_noalloc")
NOALLOC_SCRATCH_BYTES = 32 << 20   # SPECTRA_NOALLOC_SCRATCH_BYTES

_lib = None


def lib():
    """The loaded libspectra (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libspectra.so not found at {LIB_PATH}; build it first "
                               "(python spectral_transform_coding_amd/csrc/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        L.spectra_last_error.restype = ctypes.c_char_p
        L.spectra_version.restype = ctypes.c_char_p
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.spectra_calibrate.argtypes = [_PD, _PD, _PD, i32, i32, i32, ctypes.POINTER(_CalibParams),
                                        ctypes.POINTER(_CalibOut)]
        L.spectra_cache_bytes.argtypes = [ctypes.POINTER(_Layout), i32, i32, i64, ctypes.POINTER(sz)]
        L.spectra_block_bytes.argtypes = [ctypes.POINTER(_Layout), i32, ctypes.POINTER(sz)]
        L.spectra_decode_workspace_bytes.argtypes = [ctypes.POINTER(_Layout), i32, i64, ctypes.POINTER(sz)]
        L.spectra_encode_append.argtypes = [ctypes.POINTER(_Layout), i32, vp, i32, i32, vp, vp, vp,
                                            i64, _PI32, vp, vp]
        L.spectra_decode_attn.argtypes = [ctypes.POINTER(_Layout), i32, vp, vp, vp, i64, i32, _PI32,
                                          vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
        L.spectra_unpack_dequant.argtypes = [ctypes.POINTER(_Layout), i32, vp, i64, i32, i64, i64,
                                             vp, vp]
        L.spectra_decode_literal_workspace_bytes.argtypes = [ctypes.POINTER(_Layout), i32, i64, ctypes.POINTER(sz)]
        L.spectra_decode_attn_literal.argtypes = [ctypes.POINTER(_Layout), i32, vp, vp, vp, i64, i32, _PI32,
                                                  vp, vp, ctypes.c_float, vp, vp, sz, vp]
        L.spectra_decode_attn_noalloc.argtypes = [ctypes.POINTER(_Layout), i32, vp, vp, vp, i64, i32, _PI32,
                                                  vp, vp, ctypes.c_float, vp, vp, vp]
        L.spectra_set_timing_events.argtypes = [vp, vp]
        L.spectra_set_timing_events.restype = None
        L.spectra_set_jit.argtypes = [ctypes.c_int]
        L.spectra_set_jit.restype = ctypes.c_int
        L.spectra_set_key_split.argtypes = [ctypes.c_int]
        L.spectra_set_key_split.restype = ctypes.c_int
        L.spectra_jit_kernel_count.argtypes = []
        L.spectra_jit_kernel_count.restype = ctypes.c_int
        for f in SYMBOLS:
            if f not in ("spectra_last_error", "spectra_version", "spectra_set_timing_events"):
                getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        raise SpectraError(status, lib().spectra_last_error().decode())


def version():
    return lib().spectra_version().decode()


class Layout:
    """One layer's codec shape.  widths_k / widths_v: int [n_seg, seg_rank / group_size]."""

    def __init__(self, d_model, n_q_heads, n_kv_heads, d_head, n_seg, seg_rank, group_size,
                 widths_k, widths_v):
        self.d_model, self.n_q_heads, self.n_kv_heads, self.d_head = d_model, n_q_heads, n_kv_heads, d_head
        self.n_seg, self.seg_rank, self.group_size = n_seg, seg_rank, group_size
        self.widths_k = np.ascontiguousarray(np.asarray(widths_k).reshape(-1), dtype=np.uint8)
        self.widths_v = np.ascontiguousarray(np.asarray(widths_v).reshape(-1), dtype=np.uint8)
        self._c = _Layout(d_model, n_q_heads, n_kv_heads, d_head, n_seg, seg_rank, group_size,
                          self.widths_k.ctypes.data_as(_PU8), self.widths_v.ctypes.data_as(_PU8))
        self._ref = ctypes.byref(self._c)
        self._r_act = (int(np.count_nonzero(self.widths_k)) * group_size,
                       int(np.count_nonzero(self.widths_v)) * group_size)
        self._sizes = {}

    @property
    def c(self):
        return self._ref

    def r_act(self, tensor):
        return self._r_act[0 if tensor == TENSOR_K else 1]

    def cache_bytes(self, tensor, batch, cap_tokens):
        key = (int(tensor), int(batch), int(cap_tokens))
        v = self._sizes.get(key)
        if v is None:
            out = ctypes.c_size_t()
            _check(lib().spectra_cache_bytes(self.c, tensor, batch, cap_tokens, ctypes.byref(out)))
            v = self._sizes[key] = out.value
        return v

    def block_bytes(self, tensor):
        out = ctypes.c_size_t()
        _check(lib().spectra_block_bytes(self.c, tensor, ctypes.byref(out)))
        return out.value

    def workspace_bytes(self, batch, max_ctx):
        key = ("ws", int(batch), int(max_ctx))
        v = self._sizes.get(key)
        if v is None:
            out = ctypes.c_size_t()
            _check(lib().spectra_decode_workspace_bytes(self.c, batch, max_ctx, ctypes.byref(out)))
            v = self._sizes[key] = out.value
        return v

    def literal_workspace_bytes(self, batch, max_ctx):
        out = ctypes.c_size_t()
        _check(lib().spectra_decode_literal_workspace_bytes(self.c, batch, max_ctx, ctypes.byref(out)))
        return out.value


RANK_FIXED, RANK_ENERGY, RANK_GAP = 0, 1, 2


def calibrate(G, W_K, W_V, n_kv_heads, d_head, n_seg, seg_rank, group_size, budget_bits=0.0,
              fixed_width=0, energy=0.0, scale_bits=16, max_width=8, rank_rule=RANK_FIXED,
              gap_ratio=0.0, rows=None, robust=False, value_correction=False):
    """spectra_calibrate on float64 host arrays.  rank_rule: RANK_FIXED (seg_rank), RANK_ENERGY
    (the energy rank at `energy`) or RANK_GAP (trimmed at the largest eigenvalue ratio when it
    reaches gap_ratio) limits the groups that receive bits.  rows [n x d_model]: calibration
    rows for robust=True (outlier-robust eigen-pairs from the rows; G is then not used and may
    be None) and value_correction=True (least-squares value-latent correction folded into
    w_up_v).  Returns a dict
    with w_down_t_{k,v} [r_act x d_model], w_up_{k,v} [r_act x seg_cols], widths_{k,v}
    [n_seg, groups], sigma2_{k,v} [n_seg, seg_rank], theta_{k,v} [n_seg], energy_rank_{k,v}
    [n_seg]."""
    W_K = np.ascontiguousarray(W_K, dtype=np.float64)
    W_V = np.ascontiguousarray(W_V, dtype=np.float64)
    d = W_K.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.float64)
        if rows.ndim != 2 or rows.shape[1] != d:
            raise SpectraError(EINVAL, f"calibrate: rows must be [n, {d}]")
    G = None if G is None else np.ascontiguousarray(G, dtype=np.float64)
    n_all = n_kv_heads * d_head
    seg_cols = n_all // max(n_seg, 1)
    R = n_seg * seg_rank
    groups = seg_rank // max(group_size, 1)
    arr = {
        "w_down_t_k": np.zeros((R, d)), "w_down_t_v": np.zeros((R, d)),
        "w_up_k": np.zeros((R, seg_cols)), "w_up_v": np.zeros((R, seg_cols)),
        "widths_k": np.zeros(n_seg * groups, np.uint8), "widths_v": np.zeros(n_seg * groups, np.uint8),
        "sigma2_k": np.zeros(R), "sigma2_v": np.zeros(R),
        "theta_k": np.zeros(n_seg), "theta_v": np.zeros(n_seg),
        "energy_rank_k": np.zeros(n_seg, np.int32), "energy_rank_v": np.zeros(n_seg, np.int32),
    }
    out = _CalibOut()
    for k, a in arr.items():
        ct = {np.float64: _PD, np.uint8: _PU8, np.int32: _PI32}[a.dtype.type]
        setattr(out, k, a.ctypes.data_as(ct))
    p = _CalibParams(n_seg, seg_rank, group_size, float(budget_bits), int(fixed_width),
                     float(energy), scale_bits, max_width, int(rank_rule), float(gap_ratio),
                     None if rows is None else rows.ctypes.data_as(_PD),
                     0 if rows is None else rows.shape[0], int(bool(robust)), int(bool(value_correction)))
    _check(lib().spectra_calibrate(None if G is None else G.ctypes.data_as(_PD), W_K.ctypes.data_as(_PD),
                                   W_V.ctypes.data_as(_PD), d, n_kv_heads, d_head,
                                   ctypes.byref(p), ctypes.byref(out)))
    rk, rv = out.r_act_k, out.r_act_v
    res = dict(arr)
    res["w_down_t_k"] = arr["w_down_t_k"][:rk]
    res["w_down_t_v"] = arr["w_down_t_v"][:rv]
    res["w_up_k"] = arr["w_up_k"][:rk]
    res["w_up_v"] = arr["w_up_v"][:rv]
    res["widths_k"] = arr["widths_k"].reshape(n_seg, groups)
    res["widths_v"] = arr["widths_v"].reshape(n_seg, groups)
    res["sigma2_k"] = arr["sigma2_k"].reshape(n_seg, seg_rank)
    res["sigma2_v"] = arr["sigma2_v"].reshape(n_seg, seg_rank)
    res["r_act_k"], res["r_act_v"] = rk, rv
    return res


# ------------------------------------------------------------------ device calls (torch)

def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise SpectraError(EINVAL, f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _i32(values, n=None, what="array"):
    """Host int32 array of `values` as (numpy view, ctypes array passed as the pointer);
    with n given, exactly n entries."""
    vals = [int(v) for v in np.asarray(values).reshape(-1)] if isinstance(values, np.ndarray) else [int(v) for v in values]
    if n is not None and len(vals) != n:
        raise SpectraError(EINVAL, f"{what} has {len(vals)} entries, batch is {n}")
    arr = (ctypes.c_int32 * max(len(vals), 1))(*vals)
    return np.ctypeslib.as_array(arr)[:len(vals)], arr


def _nbytes(t):
    return t.numel() * t.element_size()


def _need(t, what, shape=None, dtype=None, min_bytes=None, device=None):
    """Checks one tensor argument before its pointer is passed to the library: contiguous,
    the expected shape (a tuple of ints) and dtype, at least min_bytes of storage and on the
    given device.  Raises SpectraError(EINVAL)."""
    if t is None:
        raise SpectraError(EINVAL, f"{what} is missing")
    if not t.is_contiguous():
        raise SpectraError(EINVAL, f"{what} must be contiguous")
    if shape is not None and tuple(t.shape) != shape:
        raise SpectraError(EINVAL, f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise SpectraError(EINVAL, f"{what} has dtype {t.dtype}, expected {dtype}")
    if min_bytes is not None and _nbytes(t) < min_bytes:
        raise SpectraError(EINVAL, f"{what} holds {_nbytes(t)} bytes, needs {min_bytes}")
    if device is not None and t.device != device:
        raise SpectraError(EINVAL, f"{what} is on {t.device}, expected {device}")


def _gpu_device(t, what):
    if t.device.type != "cuda":
        raise SpectraError(EINVAL, f"{what} must be on a GPU device (is on {t.device})")
    return t.device


def encode_append(layout, x, w_down_t, cache_k, cache_v, cap_tokens, start_pos,
                  latent_out=None, stream=None):
    """x [batch, n_new, d_model] (float32 or bfloat16, device), w_down_t
    [r_act_k + r_act_v, d_model] (same dtype); start_pos: host ints [batch]."""
    import torch
    if x.dim() != 3:
        raise SpectraError(EINVAL, f"x must be [batch, n_new, d_model], has shape {tuple(x.shape)}")
    batch, n_new = int(x.shape[0]), int(x.shape[1])
    code = _dtype_code(x)
    r_all = layout.r_act(TENSOR_K) + layout.r_act(TENSOR_V)
    _need(x, "x", (batch, n_new, layout.d_model))
    _need(w_down_t, "w_down_t", (r_all, layout.d_model), x.dtype)
    _need(cache_k, "cache_k", min_bytes=layout.cache_bytes(TENSOR_K, batch, cap_tokens))
    _need(cache_v, "cache_v", min_bytes=layout.cache_bytes(TENSOR_V, batch, cap_tokens))
    if latent_out is not None:
        _need(latent_out, "latent_out", dtype=torch.float32, min_bytes=batch * n_new * r_all * 4)
    sp, spp = _i32(start_pos, batch, "start_pos")
    _same_gpu(x, "x", ((w_down_t, "w_down_t"), (cache_k, "cache_k"), (cache_v, "cache_v"), (latent_out, "latent_out")))
    _check(lib().spectra_encode_append(layout.c, code, _ptr(x), batch, n_new,
                                       _ptr(w_down_t), _ptr(cache_k), _ptr(cache_v),
                                       int(cap_tokens), spp, _ptr(latent_out), _stream(stream)))


def _check_decode_args(layout, q, cache_k, cache_v, cap_tokens, w_up_k, w_up_v):
    """Shared checks of the decode calls' device arguments; returns the batch."""
    if q.dim() != 3:
        raise SpectraError(EINVAL, f"q must be [batch, n_q_heads, d_head], has shape {tuple(q.shape)}")
    batch = int(q.shape[0])
    _dtype_code(q)
    _need(q, "q", (batch, layout.n_q_heads, layout.d_head))
    seg_cols = layout.n_kv_heads * layout.d_head // max(layout.n_seg, 1)
    _need(w_up_k, "w_up_k", (layout.r_act(TENSOR_K), seg_cols), q.dtype)
    _need(w_up_v, "w_up_v", (layout.r_act(TENSOR_V), seg_cols), q.dtype)
    _need(cache_k, "cache_k", min_bytes=layout.cache_bytes(TENSOR_K, batch, cap_tokens))
    _need(cache_v, "cache_v", min_bytes=layout.cache_bytes(TENSOR_V, batch, cap_tokens))
    return batch


def _same_gpu(first, what, others):
    """All tensors on first's device, which must be a GPU (checked after everything else)."""
    dev = _gpu_device(first, what)
    for t, name in others:
        if t is not None:
            _need(t, name, device=dev)


def decode_attn(layout, q, cache_k, cache_v, cap_tokens, ctx_len, w_up_k, w_up_v,
                softmax_scale, w_o=None, out=None, workspace=None, stream=None):
    """q [batch, n_q_heads, d_head] (device); ctx_len host ints [batch].  Returns out (float32
    [batch, n_q_heads, d_head], or [batch, d_model] with w_o)."""
    import torch
    batch = _check_decode_args(layout, q, cache_k, cache_v, cap_tokens, w_up_k, w_up_v)
    cl, clp = _i32(ctx_len, batch, "ctx_len")
    shape = (batch, layout.d_model) if w_o is not None else (batch, layout.n_q_heads, layout.d_head)
    if w_o is not None:
        _need(w_o, "w_o", (layout.n_q_heads * layout.d_head, layout.d_model), q.dtype)
    if out is not None:
        _need(out, "out", shape, torch.float32)
    if workspace is not None:
        _need(workspace, "workspace")
    _same_gpu(q, "q", ((w_up_k, "w_up_k"), (w_up_v, "w_up_v"), (cache_k, "cache_k"), (cache_v, "cache_v"),
                       (w_o, "w_o"), (out, "out"), (workspace, "workspace")))
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = layout.workspace_bytes(batch, int(cl.max()) if cl.size else 0)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().spectra_decode_attn(layout.c, _dtype_code(q), _ptr(q), _ptr(cache_k), _ptr(cache_v),
                                     int(cap_tokens), batch, clp, _ptr(w_up_k), _ptr(w_up_v),
                                     float(softmax_scale), _ptr(w_o), _ptr(out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def decode_attn_noalloc(layout, q, cache_k, cache_v, cap_tokens, ctx_len, w_up_k, w_up_v,
                        softmax_scale, w_o=None, out=None, stream=None):
    """spectra_decode_attn_noalloc: decode_attn without a workspace argument; the library draws
    it from its per-device scratch (calls on one device must not overlap).  With out=None the
    output tensor is allocated here, by torch; pass `out` to allocate nothing."""
    import torch
    batch = _check_decode_args(layout, q, cache_k, cache_v, cap_tokens, w_up_k, w_up_v)
    cl, clp = _i32(ctx_len, batch, "ctx_len")
    shape = (batch, layout.d_model) if w_o is not None else (batch, layout.n_q_heads, layout.d_head)
    if w_o is not None:
        _need(w_o, "w_o", (layout.n_q_heads * layout.d_head, layout.d_model), q.dtype)
    if out is not None:
        _need(out, "out", shape, torch.float32)
    _same_gpu(q, "q", ((w_up_k, "w_up_k"), (w_up_v, "w_up_v"), (cache_k, "cache_k"), (cache_v, "cache_v"),
                       (w_o, "w_o"), (out, "out")))
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    _check(lib().spectra_decode_attn_noalloc(layout.c, _dtype_code(q), _ptr(q), _ptr(cache_k), _ptr(cache_v),
                                             int(cap_tokens), batch, clp, _ptr(w_up_k), _ptr(w_up_v),
                                             float(softmax_scale), _ptr(w_o), _ptr(out), _stream(stream)))
    return out


def decode_attn_literal(layout, q, cache_k, cache_v, cap_tokens, ctx_len, w_up_k, w_up_v,
                        softmax_scale, out=None, workspace=None, stream=None):
    """spectra_decode_attn_literal: keys and values rebuilt for every cached token, then
    attended.  Same arguments and result as decode_attn (no w_o)."""
    import torch
    batch = _check_decode_args(layout, q, cache_k, cache_v, cap_tokens, w_up_k, w_up_v)
    cl, clp = _i32(ctx_len, batch, "ctx_len")
    if out is not None:
        _need(out, "out", (batch, layout.n_q_heads, layout.d_head), torch.float32)
    if workspace is not None:
        _need(workspace, "workspace")
    _same_gpu(q, "q", ((w_up_k, "w_up_k"), (w_up_v, "w_up_v"), (cache_k, "cache_k"), (cache_v, "cache_v"),
                       (out, "out"), (workspace, "workspace")))
    if out is None:
        out = torch.empty((batch, layout.n_q_heads, layout.d_head), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = layout.literal_workspace_bytes(batch, int(cl.max()) if cl.size else 0)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().spectra_decode_attn_literal(layout.c, _dtype_code(q), _ptr(q), _ptr(cache_k), _ptr(cache_v),
                                             int(cap_tokens), batch, clp, _ptr(w_up_k), _ptr(w_up_v),
                                             float(softmax_scale), _ptr(out), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def unpack_dequant(layout, tensor, cache, cap_tokens, batch, pos0, n_tok, out=None, stream=None):
    import torch
    _need(cache, "cache", min_bytes=layout.cache_bytes(tensor, batch, cap_tokens))
    if out is None:
        out = torch.empty((batch, n_tok, layout.r_act(tensor)), dtype=torch.float32, device=cache.device)
    _need(out, "out", (batch, n_tok, layout.r_act(tensor)), torch.float32)
    _same_gpu(cache, "cache", ((out, "out"),))
    _check(lib().spectra_unpack_dequant(layout.c, tensor, _ptr(cache), int(cap_tokens), batch,
                                        int(pos0), int(n_tok), _ptr(out), _stream(stream)))
    return out


def set_timing_events(before, after):
    """Record `before`/`after` (torch.cuda.Event) around the next decode's streaming kernel."""
    lib().spectra_set_timing_events(ctypes.c_void_p(before.cuda_event) if before is not None else None,
                                    ctypes.c_void_p(after.cuda_event) if after is not None else None)


def set_jit(mode: int) -> int:
    """Run-time specialised decode kernels on (1) or off (0); other values only query.
    Returns the previous setting."""
    return int(lib().spectra_set_jit(int(mode)))


def set_key_split(mode: int) -> int:
    """Decode key-score precision on the matrix-core path: 0 splits the leading three quarters of
    the key groups into two fp16 terms (default), 1 splits every group (for tokens far beyond the
    calibration's scale); other values only query.  Returns the previous mode."""
    return int(lib().spectra_set_key_split(int(mode)))


def jit_kernel_count() -> int:
    """Specialised decode kernels compiled so far in this process."""
    return int(lib().spectra_jit_kernel_count())
