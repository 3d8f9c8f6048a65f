"""Python binding of libsinkattn (ctypes; argument marshalling only).

The functions keep the C names (``sa_rope_create``, ``sa_cache_append``,
``sa_window_attn`` ...) and take torch CUDA tensors for device buffers;
every step runs in the HIP library.  PyTorch only supplies device memory
and the current stream.  There is no CPU fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsinkattn.so")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_DTYPE, SA_ERR_ALIGN, SA_ERR_STATE, SA_ERR_RANGE, SA_ERR_HIP = range(8)
SA_BF16, SA_F32, SA_FP8 = 0, 1, 2
SA_MASK_NONE, SA_MASK_FRAME_CAUSAL = 0, 1
SA_AXIS_T, SA_AXIS_H, SA_AXIS_W = 1, 2, 4
SA_Q_INT8, SA_Q_E4M3 = 0, 1
SA_MAX_FRAMES = 64
SA_KNOB_ATTN_KERNEL, SA_KNOB_ATTN_SPLITS, SA_KNOB_PROJ_TILE = 0, 1, 2


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_STATUS_NAMES = {0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_DTYPE",
                 4: "SA_ERR_ALIGN", 5: "SA_ERR_STATE", 6: "SA_ERR_RANGE", 7: "SA_ERR_HIP"}


class sa_rope_desc(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dim_t", ctypes.c_int32), ("dim_h", ctypes.c_int32), ("dim_w", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("theta0", ctypes.c_double), ("sigma", ctypes.c_double),
                ("eps", ctypes.POINTER(ctypes.c_double)), ("jitter_axes", ctypes.c_uint32),
                ("t_scale", ctypes.c_double), ("theta", ctypes.POINTER(ctypes.c_double))]


class sa_cache_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_local", ctypes.c_int32), ("dtype", ctypes.c_int), ("k_store", ctypes.c_void_p),
                ("v_store", ctypes.c_void_p), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class sa_slot(ctypes.Structure):
    _fields_ = [("frame", ctypes.c_int64), ("t", ctypes.c_int64), ("segment", ctypes.c_int32),
                ("slot", ctypes.c_int32)]


_VP = ctypes.c_void_p
_SIGNATURES = {
    "sa_rope_tables": (ctypes.c_int, [ctypes.POINTER(sa_rope_desc), ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_double)]),
    "sa_rope_create": (ctypes.c_int, [ctypes.POINTER(sa_rope_desc), ctypes.POINTER(_VP)]),
    "sa_rope_destroy": (None, [_VP]),
    "sa_rope3d_apply": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int64, _VP]),
    "sa_cache_store_bytes": (ctypes.c_size_t, [ctypes.POINTER(sa_cache_desc)]),
    "sa_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(sa_cache_desc)]),
    "sa_set_launch_override": (ctypes.c_int, [ctypes.c_int, ctypes.c_int32]),
    "sa_cache_create": (ctypes.c_int, [ctypes.POINTER(sa_cache_desc), _VP, ctypes.POINTER(_VP)]),
    "sa_cache_destroy": (None, [_VP]),
    "sa_cache_reset": (ctypes.c_int, [_VP]),
    "sa_cache_append": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, ctypes.c_int64, _VP]),
    "sa_cache_recache": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int32, _VP]),
    "sa_cache_project_append": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, ctypes.c_int32, _VP, ctypes.c_int32,
                                               ctypes.c_int64, _VP]),
    "sa_linear": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _VP]),
    "sa_quantize_rows": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, _VP]),
    "sa_linear_q8": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, ctypes.c_int, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, _VP]),
    "sa_cache_recache_q8": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int, ctypes.c_int32, _VP]),
    "sa_cache_project_append_q8": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int,
                                                  ctypes.c_int32, _VP, ctypes.c_int32, ctypes.c_int64, _VP]),
    "sa_window_attn_sink_mass": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int32, ctypes.c_float, ctypes.c_int,
                                                _VP, ctypes.c_size_t, _VP]),
    "sa_rope_phase_coherence": (ctypes.c_int, [ctypes.POINTER(sa_rope_desc), ctypes.POINTER(ctypes.c_double),
                                               ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                               ctypes.POINTER(ctypes.c_double)]),
    "sa_window_attn_workspace": (ctypes.c_int, [_VP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "sa_window_attn": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, ctypes.c_float, ctypes.c_int, _VP,
                                      ctypes.c_size_t, _VP]),
    "sa_window_attn_noalloc": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, ctypes.c_float, ctypes.c_int, _VP]),
    "sa_cache_slots": (ctypes.c_int, [_VP, ctypes.POINTER(sa_slot), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int32)]),
    "sa_cache_read": (ctypes.c_int, [_VP, ctypes.c_int32, _VP, _VP, _VP]),
    "sa_cache_counts": (ctypes.c_int, [_VP, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]),
    "sa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_version": (ctypes.c_char_p, []),
}

_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libsinkattn.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sink_window_kv_amd.build` "
                               "(there is no fallback implementation)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def _check(status: int, fn: str):
    if status != SA_OK:
        raise SinkAttnError(status, fn, lib().sa_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    raise SinkAttnError(SA_ERR_DTYPE, "dtype", f"unsupported tensor dtype {t.dtype}")


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _rope_desc(n_heads, head_dim, dims, grid, theta0, sigma, eps, jitter_axes, t_scale=1.0, theta=None):
    """theta: optional per-head, per-axis bases [H][3] (t, h, w); replaces theta0/sigma/eps/jitter_axes."""
    d = sa_rope_desc()
    d.n_heads, d.head_dim = n_heads, head_dim
    d.dim_t, d.dim_h, d.dim_w = dims
    d.grid_h, d.grid_w = grid
    d.theta0, d.sigma = float(theta0), float(sigma)
    keep = []
    if eps is not None:
        keep.append((ctypes.c_double * n_heads)(*[float(e) for e in eps]))
        d.eps = ctypes.cast(keep[-1], ctypes.POINTER(ctypes.c_double))
    if theta is not None:
        flat = [float(x) for row in theta for x in row]
        if len(flat) != 3 * n_heads:
            raise ValueError("theta must hold 3 bases per head")
        keep.append((ctypes.c_double * (3 * n_heads))(*flat))
        d.theta = ctypes.cast(keep[-1], ctypes.POINTER(ctypes.c_double))
    d.jitter_axes = jitter_axes
    d.t_scale = float(t_scale)
    return d, keep


def sa_set_launch_override(knob: int, value: int):
    """Test / tuning hook: force a launch shape (0 = automatic); see the header."""
    _check(lib().sa_set_launch_override(knob, value), "sa_set_launch_override")


def sa_rope_tables(n_heads, head_dim, dims, grid, theta0=10000.0, sigma=0.0, eps=None,
                   jitter_axes=SA_AXIS_T, t_scale=1.0, theta=None):
    """Host-only tables: (theta_hat [H][3], freq [H][D/2]) as nested lists of floats."""
    d, _keep = _rope_desc(n_heads, head_dim, dims, grid, theta0, sigma, eps, jitter_axes, t_scale, theta)
    th = (ctypes.c_double * (n_heads * 3))()
    fr = (ctypes.c_double * (n_heads * head_dim // 2))()
    _check(lib().sa_rope_tables(ctypes.byref(d), th, fr), "sa_rope_tables")
    return ([list(th[h * 3:(h + 1) * 3]) for h in range(n_heads)],
            [list(fr[h * head_dim // 2:(h + 1) * head_dim // 2]) for h in range(n_heads)])


class Rope:
    """Owns an sa_rope handle (per-head fp64 frequency table on the device)."""

    def __init__(self, n_heads, head_dim, dims, grid, theta0=10000.0, sigma=0.0, eps=None,
                 jitter_axes=SA_AXIS_T, t_scale=1.0, theta=None):
        self.n_heads, self.head_dim, self.dims, self.grid = n_heads, head_dim, tuple(dims), tuple(grid)
        d, _keep = _rope_desc(n_heads, head_dim, dims, grid, theta0, sigma, eps, jitter_axes, t_scale, theta)
        h = _VP()
        _check(lib().sa_rope_create(ctypes.byref(d), ctypes.byref(h)), "sa_rope_create")
        self.handle = h

    @property
    def tokens_per_frame(self):
        return self.grid[0] * self.grid[1]

    def close(self):
        if self.handle:
            lib().sa_rope_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sa_rope3d_apply(rope: Rope, x, y, batch: int, n_frames: int, t0: int, stream=None):
    _check(lib().sa_rope3d_apply(rope.handle, _ptr(x), _ptr(y), _dtype_code(x), batch, n_frames, t0,
                                 _stream(stream)), "sa_rope3d_apply")


class Cache:
    """Owns an sa_cache handle plus its two device stores (torch tensors).

    dtype: torch.bfloat16, torch.float32, or torch.float8_e4m3fn for an e4m3
    cache (bf16 k, v, q and o at the boundary; k_scale / v_scale divide the
    stored values).
    """

    def __init__(self, rope: Rope, batch: int, n_sink: int, n_local: int, dtype, device="cuda",
                 k_scale: float = 1.0, v_scale: float = 1.0):
        import torch
        if dtype == torch.float8_e4m3fn:
            code, elem = SA_FP8, 1
        else:
            code, elem = (SA_BF16, 2) if dtype == torch.bfloat16 else (SA_F32, 4)
        d = sa_cache_desc()
        d.batch, d.n_heads, d.head_dim = batch, rope.n_heads, rope.head_dim
        d.tokens_per_frame, d.n_sink, d.n_local, d.dtype = rope.tokens_per_frame, n_sink, n_local, code
        d.k_scale, d.v_scale = float(k_scale), float(v_scale)
        nbytes = lib().sa_cache_store_bytes(ctypes.byref(d))
        if nbytes == 0:
            raise SinkAttnError(SA_ERR_SHAPE, "sa_cache_store_bytes", "invalid cache descriptor")
        store_dtype = torch.uint8 if code == SA_FP8 else dtype
        self.k_store = torch.empty(nbytes // elem, dtype=store_dtype, device=device)
        self.v_store = torch.empty(nbytes // elem, dtype=store_dtype, device=device)
        d.k_store, d.v_store = self.k_store.data_ptr(), self.v_store.data_ptr()
        h = _VP()
        _check(lib().sa_cache_create(ctypes.byref(d), rope.handle, ctypes.byref(h)), "sa_cache_create")
        self.handle = h
        self.rope = rope
        self.batch, self.n_sink, self.n_local, self.dtype = batch, n_sink, n_local, dtype

    def close(self):
        if self.handle:
            lib().sa_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sa_cache_reset(cache: Cache):
    _check(lib().sa_cache_reset(cache.handle), "sa_cache_reset")


def sa_cache_append(cache: Cache, k, v, n_frames: int, t0: int, stream=None):
    _check(lib().sa_cache_append(cache.handle, _ptr(k), _ptr(v), n_frames, t0, _stream(stream)),
           "sa_cache_append")


def sa_cache_recache(cache: Cache, x, w_k, w_v, hidden: int, stream=None):
    """w_k, w_v in the [H*D, hidden] (nn.Linear) layout."""
    _check(lib().sa_cache_recache(cache.handle, _ptr(x), _ptr(w_k), _ptr(w_v), hidden, _stream(stream)),
           "sa_cache_recache")


def sa_cache_project_append(cache: Cache, x, w_q, w_k, w_v, hidden: int, q_out, n_frames: int, t0: int,
                            stream=None):
    """q_out = x . w_q^T (un-rotated); k = x . w_k^T, v = x . w_v^T appended at t0...; weights [H*D, hidden].

    w_q and q_out may both be None (cache only).
    """
    _check(lib().sa_cache_project_append(cache.handle, _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), hidden,
                                         _ptr(q_out), n_frames, t0, _stream(stream)), "sa_cache_project_append")


def sa_linear(x, w, y, n_rows: int, in_features: int, out_features: int, stream=None):
    """y [n_rows, out] = x [n_rows, in] . w^T, w in the [out, in] layout."""
    _check(lib().sa_linear(_ptr(x), _ptr(w), _ptr(y), _dtype_code(x), n_rows, in_features, out_features,
                           _stream(stream)), "sa_linear")


def sa_quantize_rows(x, codes, scales, qtype: int, stream=None):
    """Row-wise 8-bit codes of x [n_rows, n_cols] bf16: codes (int8 / uint8 bytes) same shape, scales [n_rows] fp32."""
    n_rows, n_cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (x.numel() // x.shape[-1], x.shape[-1])
    _check(lib().sa_quantize_rows(_ptr(x), _ptr(codes), _ptr(scales), qtype, n_rows, n_cols, _stream(stream)),
           "sa_quantize_rows")


def sa_linear_q8(x_codes, x_scales, w_codes, w_scales, y, qtype: int, n_rows: int, in_features: int,
                 out_features: int, stream=None):
    """y [n_rows, out] bf16 = (float(x_codes . w_codes^T) * x_scales[row]) * w_scales[feature]."""
    _check(lib().sa_linear_q8(_ptr(x_codes), _ptr(x_scales), _ptr(w_codes), _ptr(w_scales), _ptr(y), qtype, n_rows,
                              in_features, out_features, _stream(stream)), "sa_linear_q8")


def sa_cache_recache_q8(cache: Cache, x_codes, x_scales, wk_codes, wk_scales, wv_codes, wv_scales, qtype: int,
                        hidden: int, stream=None):
    """sa_cache_recache with 8-bit operands (scales per token and per output feature)."""
    _check(lib().sa_cache_recache_q8(cache.handle, _ptr(x_codes), _ptr(x_scales), _ptr(wk_codes), _ptr(wk_scales),
                                     _ptr(wv_codes), _ptr(wv_scales), qtype, hidden, _stream(stream)),
           "sa_cache_recache_q8")


def sa_cache_project_append_q8(cache: Cache, x_codes, x_scales, wq_codes, wq_scales, wk_codes, wk_scales, wv_codes,
                               wv_scales, qtype: int, hidden: int, q_out, n_frames: int, t0: int, stream=None):
    """sa_cache_project_append with 8-bit operands; wq_codes, wq_scales and q_out may all be None."""
    _check(lib().sa_cache_project_append_q8(cache.handle, _ptr(x_codes), _ptr(x_scales), _ptr(wq_codes),
                                            _ptr(wq_scales), _ptr(wk_codes), _ptr(wk_scales), _ptr(wv_codes),
                                            _ptr(wv_scales), qtype, hidden, _ptr(q_out), n_frames, t0,
                                            _stream(stream)), "sa_cache_project_append_q8")


def sa_window_attn_workspace(cache: Cache, n_q: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sa_window_attn_workspace(cache.handle, n_q, ctypes.byref(n)), "sa_window_attn_workspace")
    return n.value


def sa_window_attn(cache: Cache, q, o, n_q: int, scale: float = 0.0, mask: int = SA_MASK_NONE,
                   workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sa_window_attn(cache.handle, _ptr(q), _ptr(o), n_q, scale, mask, _ptr(workspace),
                                ws_bytes, _stream(stream)), "sa_window_attn")


def sa_window_attn_noalloc(cache: Cache, q, o, n_q: int, scale: float = 0.0, mask: int = SA_MASK_NONE,
                           stream=None):
    """sa_window_attn with the key-split partials in the library's own device scratch (no workspace)."""
    _check(lib().sa_window_attn_noalloc(cache.handle, _ptr(q), _ptr(o), n_q, scale, mask, _stream(stream)),
           "sa_window_attn_noalloc")


def sa_window_attn_sink_mass(cache: Cache, q, o, sink_mass, n_q: int, scale: float = 0.0,
                             mask: int = SA_MASK_NONE, workspace=None, stream=None):
    """o as sa_window_attn; sink_mass [B, n_q*T_f, H] float32 = softmax mass on the sink-frame keys."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sa_window_attn_sink_mass(cache.handle, _ptr(q), _ptr(o), _ptr(sink_mass), n_q, scale, mask,
                                          _ptr(workspace), ws_bytes, _stream(stream)), "sa_window_attn_sink_mass")


def sa_rope_phase_coherence(n_heads, head_dim, dims, grid, deltas: Sequence[float], theta0=10000.0, sigma=0.0,
                            eps=None, jitter_axes=SA_AXIS_T, t_scale=1.0, theta=None):
    """Host-only C_h(delta) over each head's time-axis frequencies: list (per head) of complex values."""
    d, _keep = _rope_desc(n_heads, head_dim, dims, grid, theta0, sigma, eps, jitter_axes, t_scale, theta)
    n = len(deltas)
    dl = (ctypes.c_double * max(n, 1))(*[float(x) for x in deltas])
    re = (ctypes.c_double * max(n_heads * n, 1))()
    im = (ctypes.c_double * max(n_heads * n, 1))()
    _check(lib().sa_rope_phase_coherence(ctypes.byref(d), dl, n, re, im), "sa_rope_phase_coherence")
    return [[complex(re[h * n + k], im[h * n + k]) for k in range(n)] for h in range(n_heads)]


def sa_cache_slots(cache: Cache) -> List[sa_slot]:
    n = ctypes.c_int32()
    buf = (sa_slot * SA_MAX_FRAMES)()
    _check(lib().sa_cache_slots(cache.handle, buf, SA_MAX_FRAMES, ctypes.byref(n)), "sa_cache_slots")
    return [buf[i] for i in range(n.value)]


def sa_cache_read(cache: Cache, index: int, k_out=None, v_out=None, stream=None):
    _check(lib().sa_cache_read(cache.handle, index, _ptr(k_out), _ptr(v_out), _stream(stream)),
           "sa_cache_read")


def sa_cache_counts(cache: Cache):
    a = ctypes.c_int64()
    r = ctypes.c_int32()
    _check(lib().sa_cache_counts(cache.handle, ctypes.byref(a), ctypes.byref(r)), "sa_cache_counts")
    return a.value, r.value


def sa_version() -> str:
    return lib().sa_version().decode()
