"""Python binding of libfsa (ctypes). Argument marshalling only: every step of
the computation runs in the HIP library; torch supplies device memory and the
current stream.

Signatures mirror include/fsa.h: tensors are contiguous [B, H, N, 64] in
float32 or bfloat16 on one GPU; LSE and the backward D workspace are float32
[B, H, N]; the backward pair workspace is a device buffer of
workspace_bytes(...) bytes (allocated here when the caller passes none). There
is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfsa.so")

FSA_OK, FSA_E_ARG, FSA_E_UNSUPPORTED, FSA_E_CAPACITY, FSA_E_HIP = range(5)
STATUS_NAMES = {0: "FSA_OK", 1: "FSA_E_ARG", 2: "FSA_E_UNSUPPORTED", 3: "FSA_E_CAPACITY", 4: "FSA_E_HIP"}
BASES = {"fib": 0, "pow2": 1}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
MAX_OFFSETS = 48

# Exported symbols, in the order include/fsa.h declares them.
EXPORTS = ("fsa_build_offsets", "fsa_forward", "fsa_backward", "fsa_backward_workspace_bytes",
           "fsa_backward_delta", "fsa_backward_grads", "fsa_decode", "fsa_dense_forward",
           "fsa_frac_offsets", "fsa_frac_forward", "fsa_frac_backward", "fsa_frac_backward_workspace_bytes",
           "fsa_frac_decode",
           "fsa_rope_table", "fsa_rope_rotate", "fsa_rope_workspace_bytes", "fsa_rope_forward", "fsa_rope_backward",
           "fsa_rope_frac_workspace_bytes", "fsa_rope_frac_forward", "fsa_rope_frac_backward", "fsa_wait_status",
           "fsa_backward_noalloc", "fsa_debug_force_wait_timeout", "fsa_debug_tile_order", "fsa_last_error")
WS_KINDS = {"backward": 0, "frac_backward": 1, "rope_backward": 2, "rope_frac_backward": 3, "backward_noalloc": 4,
            "rope_forward": 5}


class FsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()


def library() -> ctypes.CDLL:
    """Loads libfsa.so from the package directory (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise FsaError(-1, f"{_LIB_PATH} is missing; build it with "
                                   "`python -m fibonacci_offset_transformer_amd.build`")
            L = ctypes.CDLL(_LIB_PATH)
            i32, f32, f64, vp = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
            L.fsa_build_offsets.argtypes = [ctypes.c_int, f64, i32, i32, ctypes.POINTER(i32), i32,
                                            ctypes.POINTER(i32)]
            L.fsa_build_offsets.restype = ctypes.c_int
            L.fsa_forward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                      ctypes.c_int, f64, i32, i32, vp]
            L.fsa_forward.restype = ctypes.c_int
            u64 = ctypes.c_uint64
            L.fsa_backward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64,
                                       i32, i32, i32, i32, f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_backward.restype = ctypes.c_int
            L.fsa_backward_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, ctypes.c_int, f64, i32,
                                                       i32, ctypes.POINTER(u64)]
            L.fsa_backward_workspace_bytes.restype = ctypes.c_int
            L.fsa_backward_delta.argtypes = [ctypes.c_int, vp, vp, vp, i32, i32, i32, i32, vp]
            L.fsa_backward_delta.restype = ctypes.c_int
            L.fsa_backward_grads.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64,
                                             i32, i32, i32, i32, f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_backward_grads.restype = ctypes.c_int
            L.fsa_decode.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                     ctypes.c_int, f64, i32, i32, vp]
            L.fsa_decode.restype = ctypes.c_int
            L.fsa_dense_forward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
            L.fsa_dense_forward.restype = ctypes.c_int
            L.fsa_frac_offsets.argtypes = [ctypes.c_int, f64, i32, i32, ctypes.POINTER(i32),
                                           ctypes.POINTER(f32), ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]
            L.fsa_frac_offsets.restype = ctypes.c_int
            L.fsa_frac_forward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                           f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_frac_forward.restype = ctypes.c_int
            L.fsa_frac_backward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, u64, i32, i32, i32, i32, f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_frac_backward.restype = ctypes.c_int
            L.fsa_frac_backward_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, ctypes.c_int, f64,
                                                            i32, i32, ctypes.POINTER(u64)]
            L.fsa_frac_backward_workspace_bytes.restype = ctypes.c_int
            L.fsa_frac_decode.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                          f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_frac_decode.restype = ctypes.c_int
            L.fsa_rope_table.argtypes = [i32, i32, f64, ctypes.POINTER(f32)]
            L.fsa_rope_table.restype = ctypes.c_int
            L.fsa_rope_rotate.argtypes = [ctypes.c_int, vp, vp, i32, vp, i32, i32, i32, i32, vp]
            L.fsa_rope_rotate.restype = ctypes.c_int
            L.fsa_rope_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, ctypes.c_int, f64, i32, i32,
                                                   ctypes.POINTER(u64), ctypes.POINTER(u64)]
            L.fsa_rope_workspace_bytes.restype = ctypes.c_int
            L.fsa_rope_forward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i32, vp, vp, vp, u64, i32, i32,
                                           i32, i32, i32, f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_rope_forward.restype = ctypes.c_int
            L.fsa_rope_backward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                            u64, i32, i32, i32, i32, i32, f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_rope_backward.restype = ctypes.c_int
            L.fsa_rope_frac_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, ctypes.c_int, f64, i32,
                                                        i32, ctypes.POINTER(u64), ctypes.POINTER(u64)]
            L.fsa_rope_frac_workspace_bytes.restype = ctypes.c_int
            L.fsa_rope_frac_forward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i32, vp, vp, vp, u64, i32,
                                                i32, i32, i32, f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_rope_frac_forward.restype = ctypes.c_int
            L.fsa_rope_frac_backward.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                                 vp, vp, vp, vp, u64, i32, i32, i32, i32, i32, f32, ctypes.c_int, f64,
                                                 i32, i32, vp]
            L.fsa_rope_frac_backward.restype = ctypes.c_int
            L.fsa_wait_status.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, i32, i32, ctypes.c_int, f64, i32, i32,
                                          vp, u64, ctypes.POINTER(i32), vp]
            L.fsa_wait_status.restype = ctypes.c_int
            L.fsa_backward_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                               i32, i32, i32, f32, ctypes.c_int, f64, i32, i32, vp]
            L.fsa_backward_noalloc.restype = ctypes.c_int
            L.fsa_debug_force_wait_timeout.argtypes = [i32]
            L.fsa_debug_force_wait_timeout.restype = ctypes.c_int
            L.fsa_debug_tile_order.argtypes = [i32, ctypes.POINTER(i32)]
            L.fsa_debug_tile_order.restype = ctypes.c_int
            L.fsa_last_error.argtypes = []
            L.fsa_last_error.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(status: int) -> None:
    if status != FSA_OK:
        raise FsaError(status, library().fsa_last_error().decode())


def build_offsets(alpha: float, w: int, R: int, base: str = "fib") -> list[int]:
    """Sparse offset table of one layer (host call; see fsa_build_offsets)."""
    L = library()
    out = (ctypes.c_int32 * MAX_OFFSETS)()
    count = ctypes.c_int32(0)
    _check(L.fsa_build_offsets(BASES[base], float(alpha), int(w), int(R), out, MAX_OFFSETS,
                               ctypes.byref(count)))
    return [int(out[t]) for t in range(count.value)]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _shape(q: torch.Tensor, *others: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    if q.dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (q,) + others:
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("all tensors must share shape, dtype and device")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous CUDA/HIP tensors")
    return q.shape


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def _out(like, out, out_dtype):
    if out is None:
        return torch.empty_like(like, dtype=out_dtype or like.dtype)
    if out.shape != like.shape or not out.is_contiguous() or out.device != like.device:
        raise ValueError("output must be a contiguous tensor of the input shape on the same device")
    if out_dtype is not None and out.dtype != out_dtype:
        raise ValueError("output dtype does not match out_dtype")
    return out


def _rows(like, t, name, shape=None):
    """Per-row float32 buffer (LSE or D): the caller's tensor, checked, or a new one.
    shape defaults to like's [B, H, N]."""
    shape = tuple(like.shape[:3]) if shape is None else tuple(shape)
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() or t.device != like.device:
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {list(shape)} on the inputs' device")
    return t


def _rows_in(like, t, name):
    """A per-row float32 input (LSE, or D): must be given, [B, H, N], contiguous, on the inputs' device."""
    if t is None:
        raise ValueError(f"{name} is required")
    return _rows(like, t, name)


def forward(q, k, v, *, alpha: float = 1.0, w: int, R: int, base: str = "fib", scale=None,
            out=None, lse=None, out_dtype=None):
    """Sparse forward: returns (o [B,H,N,d] in out_dtype (default q.dtype), lse [B,H,N] float32)."""
    B, H, N, d = _shape(q, k, v)
    o = _out(q, out, out_dtype)
    l = _rows(q, lse, "lse")
    with torch.cuda.device(q.device):
        _check(library().fsa_forward(DTYPES[q.dtype], DTYPES[o.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l),
                                     B, H, N, d, _scale(scale, d), BASES[base], float(alpha), int(w),
                                     int(R), _stream(q.device)))
    return o, l


def workspace_bytes(dtype, B: int, H: int, N: int, d: int = 64, *, alpha: float = 1.0, w: int, R: int,
                    base: str = "fib") -> int:
    """Bytes of pair workspace the backward of this problem needs (see fsa_backward_workspace_bytes)."""
    out = ctypes.c_uint64(0)
    _check(library().fsa_backward_workspace_bytes(DTYPES[dtype], int(B), int(H), int(N), int(d), BASES[base],
                                                  float(alpha), int(w), int(R), ctypes.byref(out)))
    return int(out.value)


def _pair_ws(q, pair_ws, alpha, w, R, base):
    """(pointer, size) of the pair workspace: the caller's buffer, or a new one of the size needed."""
    B, H, N, d = q.shape
    if pair_ws is None:
        need = workspace_bytes(q.dtype, B, H, N, d, alpha=alpha, w=w, R=R, base=base)
        if need == 0:
            return None, 0
        pair_ws = torch.empty(need // 4, dtype=torch.int32, device=q.device)
    if not pair_ws.is_cuda or not pair_ws.is_contiguous() or pair_ws.device != q.device:
        raise ValueError("pair_ws must be a contiguous device tensor on the inputs' device")
    return pair_ws, pair_ws.numel() * pair_ws.element_size()


def backward(q, k, v, o, lse, dout, *, alpha: float = 1.0, w: int, R: int, base: str = "fib",
             scale=None, dq=None, dk=None, dv=None, delta=None, pair_ws=None, out_dtype=None):
    """Sparse backward: returns (dq, dk, dv) in out_dtype (default q.dtype).
    q, k, v, o and dout share one dtype."""
    B, H, N, d = _shape(q, k, v, o, dout)
    dq = _out(q, dq, out_dtype)
    dk = _out(q, dk, dq.dtype)
    dv = _out(q, dv, dq.dtype)
    lse = _rows_in(q, lse, "lse")
    ws = _rows(q, delta, "delta")
    pw, pw_bytes = _pair_ws(q, pair_ws, alpha, w, R, base)
    with torch.cuda.device(q.device):
        _check(library().fsa_backward(DTYPES[q.dtype], DTYPES[dq.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), _ptr(pw), pw_bytes,
                                      B, H, N, d, _scale(scale, d), BASES[base], float(alpha), int(w), int(R),
                                      _stream(q.device)))
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, dout, *, alpha: float = 1.0, w: int, R: int, base: str = "fib",
                     scale=None, dq=None, dk=None, dv=None, out_dtype=None):
    """backward() with the workspaces in the library's static device scratch (see
    fsa_backward_noalloc): the C call allocates nothing. Outputs are allocated here only
    when not given."""
    B, H, N, d = _shape(q, k, v, o, dout)
    lse = _rows_in(q, lse, "lse")
    dq = _out(q, dq, out_dtype)
    dk = _out(q, dk, dq.dtype)
    dv = _out(q, dv, dq.dtype)
    with torch.cuda.device(q.device):
        _check(library().fsa_backward_noalloc(DTYPES[q.dtype], DTYPES[dq.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                              _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                                              _scale(scale, d), BASES[base], float(alpha), int(w), int(R),
                                              _stream(q.device)))
    return dq, dk, dv


def backward_delta(o, dout, *, delta=None):
    """First backward stage: D = rowsum(dout * o), float32 [B, H, N]."""
    B, H, N, d = _shape(o, dout)
    ws = _rows(o, delta, "delta")
    with torch.cuda.device(o.device):
        _check(library().fsa_backward_delta(DTYPES[o.dtype], _ptr(o), _ptr(dout), _ptr(ws), B, H, N, d,
                                            _stream(o.device)))
    return ws


def backward_grads(q, k, v, lse, dout, delta, *, alpha: float = 1.0, w: int, R: int, base: str = "fib",
                   scale=None, dq=None, dk=None, dv=None, pair_ws=None, out_dtype=None):
    """Second backward stage: (dq, dk, dv) from a D computed by backward_delta."""
    B, H, N, d = _shape(q, k, v, dout)
    lse = _rows_in(q, lse, "lse")
    delta = _rows_in(q, delta, "delta")
    dq = _out(q, dq, out_dtype)
    dk = _out(q, dk, dq.dtype)
    dv = _out(q, dv, dq.dtype)
    pw, pw_bytes = _pair_ws(q, pair_ws, alpha, w, R, base)
    with torch.cuda.device(q.device):
        _check(library().fsa_backward_grads(DTYPES[q.dtype], DTYPES[dq.dtype], _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(lse), _ptr(dout), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                                            _ptr(pw), pw_bytes, B, H, N, d, _scale(scale, d), BASES[base],
                                            float(alpha), int(w), int(R), _stream(q.device)))
    return dq, dk, dv


def decode(q, k_cache, v_cache, seq_lens, *, alpha: float = 1.0, w: int, R: int, base: str = "fib", scale=None,
           out=None, lse=None, out_dtype=None, fractional: bool = False):
    """One decoding step: q [B,H,d] (the newest token of each sequence) against
    k_cache, v_cache [B,H,Lmax,d] with seq_lens int32 [B] on the device. Returns
    (o [B,H,d] in out_dtype (default q.dtype), lse [B,H] float32). With fractional,
    the learned-alpha variant's interpolated entries (fsa_frac_decode)."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("expected q [B, H, d] and caches [B, H, Lmax, d]")
    B, H, d = q.shape
    Lmax = k_cache.shape[2]
    for t in (k_cache, v_cache):
        if t.shape != (B, H, Lmax, d) or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("caches must be contiguous [B, H, Lmax, d] tensors of q's dtype and device")
    if q.dtype not in DTYPES or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 or bfloat16 device tensor")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or seq_lens.device != q.device:
        raise ValueError("seq_lens must be an int32 [B] tensor on q's device")
    o = _out(q, out, out_dtype)
    l = _rows(q, lse, "lse", (B, H))
    fn = library().fsa_frac_decode if fractional else library().fsa_decode
    with torch.cuda.device(q.device):
        _check(fn(DTYPES[q.dtype], DTYPES[o.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(o),
                  _ptr(l), B, H, Lmax, d, _scale(scale, d), BASES[base], float(alpha), int(w), int(R),
                  _stream(q.device)))
    return o, l


def dense_forward(q, k, v, *, scale=None, out=None, lse=None, out_dtype=None):
    """Dense causal baseline: returns (o, lse)."""
    B, H, N, d = _shape(q, k, v)
    o = _out(q, out, out_dtype)
    l = _rows(q, lse, "lse")
    with torch.cuda.device(q.device):
        _check(library().fsa_dense_forward(DTYPES[q.dtype], DTYPES[o.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l),
                                           B, H, N, d, _scale(scale, d), _stream(q.device)))
    return o, l


# ----------------------------------------------------------------------------
# learned-alpha variant: fractional entries
# ----------------------------------------------------------------------------


def frac_offsets(alpha: float, w: int, R: int, base: str = "fib") -> list[tuple[int, float, int]]:
    """Fractional table of one layer: [(floor(d), d - floor(d) as float, F)] (see fsa_frac_offsets)."""
    L = library()
    whole = (ctypes.c_int32 * MAX_OFFSETS)()
    frac = (ctypes.c_float * MAX_OFFSETS)()
    fb = (ctypes.c_int32 * MAX_OFFSETS)()
    count = ctypes.c_int32(0)
    _check(L.fsa_frac_offsets(BASES[base], float(alpha), int(w), int(R), whole, frac, fb, MAX_OFFSETS,
                              ctypes.byref(count)))
    return [(int(whole[t]), float(frac[t]), int(fb[t])) for t in range(count.value)]


def frac_forward(q, k, v, *, alpha: float, w: int, R: int, base: str = "fib", scale=None, out=None, lse=None,
                 out_dtype=None):
    """Learned-alpha forward (interpolated entries): returns (o, lse) like forward()."""
    B, H, N, d = _shape(q, k, v)
    o = _out(q, out, out_dtype)
    l = _rows(q, lse, "lse")
    with torch.cuda.device(q.device):
        _check(library().fsa_frac_forward(DTYPES[q.dtype], DTYPES[o.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                          _ptr(l), B, H, N, d, _scale(scale, d), BASES[base], float(alpha), int(w),
                                          int(R), _stream(q.device)))
    return o, l


def frac_workspace_bytes(dtype, B: int, H: int, N: int, d: int = 64, *, alpha: float, w: int, R: int,
                         base: str = "fib") -> int:
    """Bytes of workspace fsa_frac_backward needs for this problem."""
    out = ctypes.c_uint64(0)
    _check(library().fsa_frac_backward_workspace_bytes(DTYPES[dtype], int(B), int(H), int(N), int(d),
                                                       BASES[base], float(alpha), int(w), int(R),
                                                       ctypes.byref(out)))
    return int(out.value)


def frac_backward(q, k, v, o, lse, dout, *, alpha: float, w: int, R: int, base: str = "fib", scale=None,
                  dq=None, dk=None, dv=None, dalpha=None, doffs=None, ws=None, out_dtype=None):
    """Learned-alpha backward: returns (dq, dk, dv, dalpha float32 [1], doffs float32 [entries]).
    ws is the device workspace (allocated here when not given)."""
    B, H, N, d = _shape(q, k, v, o, dout)
    lse = _rows_in(q, lse, "lse")
    dq = _out(q, dq, out_dtype)
    dk = _out(q, dk, dq.dtype)
    dv = _out(q, dv, dq.dtype)
    n_entries = len(frac_offsets(alpha, w, R, base))
    if dalpha is None:
        dalpha = torch.empty(1, dtype=torch.float32, device=q.device)
    if doffs is None:
        doffs = torch.empty(max(n_entries, 1), dtype=torch.float32, device=q.device)
    for t, n in ((dalpha, 1), (doffs, n_entries)):
        if t.dtype != torch.float32 or t.device != q.device or not t.is_contiguous() or t.numel() < n:
            raise ValueError("dalpha and doffs must be contiguous float32 device tensors of sufficient size")
    if ws is None:
        need = frac_workspace_bytes(q.dtype, B, H, N, d, alpha=alpha, w=w, R=R, base=base)
        ws = torch.empty(max(need // 4, 1), dtype=torch.int32, device=q.device)
    if not ws.is_cuda or not ws.is_contiguous() or ws.device != q.device:
        raise ValueError("ws must be a contiguous device tensor on the inputs' device")
    with torch.cuda.device(q.device):
        _check(library().fsa_frac_backward(DTYPES[q.dtype], DTYPES[dq.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                           _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha),
                                           _ptr(doffs), _ptr(ws), ws.numel() * ws.element_size(), B, H, N, d,
                                           _scale(scale, d), BASES[base], float(alpha), int(w), int(R),
                                           _stream(q.device)))
    return dq, dk, dv, dalpha, doffs[:n_entries]


# ----------------------------------------------------------------------------
# rotary position embedding before the attention
# ----------------------------------------------------------------------------


def rope_table(n_pos: int, d: int = 64, rope_base: float = 10000.0, device=None) -> torch.Tensor:
    """Rotary table [n_pos, d/2, 2] float32 (cos, sin) built on the host by fsa_rope_table;
    returned on `device` (host when None)."""
    host = torch.empty((max(int(n_pos), 0), int(d) // 2, 2), dtype=torch.float32)
    ptr = ctypes.cast(host.data_ptr(), ctypes.POINTER(ctypes.c_float)) if host.numel() else None
    _check(library().fsa_rope_table(int(n_pos), int(d), float(rope_base), ptr))
    return host if device is None else host.to(device)


def _table(table, N):
    if table.dtype != torch.float32 or not table.is_cuda or not table.is_contiguous() or table.dim() != 3:
        raise ValueError("the rotary table must be a contiguous float32 [n_pos, d/2, 2] device tensor")
    return int(table.shape[0])


def rope_rotate(x, table, *, out=None):
    """The rotation step alone: bf16 [B,H,N,d] -> bf16 rotated rows."""
    B, H, N, d = _shape(x)
    y = _out(x, out, x.dtype)
    n_pos = _table(table, N)
    with torch.cuda.device(x.device):
        _check(library().fsa_rope_rotate(DTYPES[x.dtype], _ptr(x), _ptr(table), n_pos, _ptr(y), B, H, N, d,
                                         _stream(x.device)))
    return y


def rope_workspace_bytes(dtype, B: int, H: int, N: int, d: int = 64, *, alpha: float = 1.0, w: int, R: int,
                         base: str = "fib") -> tuple[int, int]:
    """(forward, backward) workspace bytes of the rotary calls."""
    f, b = ctypes.c_uint64(0), ctypes.c_uint64(0)
    _check(library().fsa_rope_workspace_bytes(DTYPES[dtype], int(B), int(H), int(N), int(d), BASES[base],
                                              float(alpha), int(w), int(R), ctypes.byref(f), ctypes.byref(b)))
    return int(f.value), int(b.value)


def _rope_ws(q, ws, which, alpha, w, R, base):
    B, H, N, d = q.shape
    need = rope_workspace_bytes(q.dtype, B, H, N, d, alpha=alpha, w=w, R=R, base=base)[which]
    if ws is None:
        ws = torch.empty(max(need // 4, 4), dtype=torch.int32, device=q.device)
    if not ws.is_cuda or not ws.is_contiguous() or ws.device != q.device:
        raise ValueError("ws must be a contiguous device tensor on the inputs' device")
    return ws, ws.numel() * ws.element_size()


def rope_forward(q, k, v, table, *, alpha: float = 1.0, w: int, R: int, base: str = "fib", scale=None, out=None,
                 lse=None, out_dtype=None, ws=None, keep_rotated: bool = True):
    """Forward on rotated Q, K (unrotated inputs, rotary table on the device): (o, lse).
    keep_rotated leaves the rotated Q in ws beside the rotated K for rope_backward's
    reuse_rotated; inference can pass False."""
    B, H, N, d = _shape(q, k, v)
    o = _out(q, out, out_dtype)
    l = _rows(q, lse, "lse")
    n_pos = _table(table, N)
    ws, ws_bytes = _rope_ws(q, ws, 0, alpha, w, R, base)
    with torch.cuda.device(q.device):
        _check(library().fsa_rope_forward(DTYPES[q.dtype], DTYPES[o.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(table),
                                          n_pos, _ptr(o), _ptr(l), _ptr(ws), ws_bytes, int(bool(keep_rotated)), B, H, N,
                                          d, _scale(scale, d), BASES[base], float(alpha), int(w), int(R),
                                          _stream(q.device)))
    return o, l


def rope_backward(q, k, v, table, o, lse, dout, *, alpha: float = 1.0, w: int, R: int, base: str = "fib",
                  scale=None, dq=None, dk=None, dv=None, out_dtype=None, ws=None, reuse_rotated: bool = False):
    """Backward of rope_forward: (dq, dk, dv) with respect to the unrotated inputs. With
    reuse_rotated, ws must still hold the rotated rows rope_forward wrote for these q, k."""
    if reuse_rotated and ws is None:
        raise ValueError("reuse_rotated needs the forward's workspace")
    B, H, N, d = _shape(q, k, v, o, dout)
    lse = _rows_in(q, lse, "lse")
    dq = _out(q, dq, out_dtype)
    dk = _out(q, dk, dq.dtype)
    dv = _out(q, dv, dq.dtype)
    n_pos = _table(table, N)
    ws, ws_bytes = _rope_ws(q, ws, 1, alpha, w, R, base)
    with torch.cuda.device(q.device):
        _check(library().fsa_rope_backward(DTYPES[q.dtype], DTYPES[dq.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(table),
                                           n_pos, _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                           _ptr(ws), ws_bytes, int(bool(reuse_rotated)), B, H, N, d, _scale(scale, d),
                                           BASES[base], float(alpha), int(w), int(R), _stream(q.device)))
    return dq, dk, dv


# ---- RoPE before the gather, then the learned-alpha variant ----


def rope_frac_workspace_bytes(dtype, B: int, H: int, N: int, d: int = 64, *, alpha: float, w: int, R: int,
                              base: str = "fib") -> tuple[int, int]:
    """(forward, backward) workspace bytes of the rotary learned-alpha calls."""
    f, b = ctypes.c_uint64(0), ctypes.c_uint64(0)
    _check(library().fsa_rope_frac_workspace_bytes(DTYPES[dtype], int(B), int(H), int(N), int(d), BASES[base],
                                                   float(alpha), int(w), int(R), ctypes.byref(f), ctypes.byref(b)))
    return int(f.value), int(b.value)


def rope_frac_forward(q, k, v, table, *, alpha: float, w: int, R: int, base: str = "fib", scale=None, out=None,
                      lse=None, out_dtype=None, ws=None):
    """Learned-alpha forward over rotated Q, K (unrotated inputs): (o, lse)."""
    B, H, N, d = _shape(q, k, v)
    o = _out(q, out, out_dtype)
    l = _rows(q, lse, "lse")
    n_pos = _table(table, N)
    if ws is None:
        need = rope_frac_workspace_bytes(q.dtype, B, H, N, d, alpha=alpha, w=w, R=R, base=base)[0]
        ws = torch.empty(max(need // 4, 4), dtype=torch.int32, device=q.device)
    with torch.cuda.device(q.device):
        _check(library().fsa_rope_frac_forward(DTYPES[q.dtype], DTYPES[o.dtype], _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(table), n_pos, _ptr(o), _ptr(l), _ptr(ws),
                                               ws.numel() * ws.element_size(), B, H, N, d, _scale(scale, d),
                                               BASES[base], float(alpha), int(w), int(R), _stream(q.device)))
    return o, l


def rope_frac_backward(q, k, v, table, o, lse, dout, *, alpha: float, w: int, R: int, base: str = "fib",
                       scale=None, dq=None, dk=None, dv=None, dalpha=None, doffs=None, out_dtype=None, ws=None,
                       reuse_rotated: bool = False):
    """Backward of rope_frac_forward: (dq, dk, dv, dalpha [1], doffs [entries])."""
    B, H, N, d = _shape(q, k, v, o, dout)
    lse = _rows_in(q, lse, "lse")
    dq = _out(q, dq, out_dtype)
    dk = _out(q, dk, dq.dtype)
    dv = _out(q, dv, dq.dtype)
    n_pos = _table(table, N)
    n_entries = len(frac_offsets(alpha, w, R, base))
    dalpha = torch.empty(1, dtype=torch.float32, device=q.device) if dalpha is None else dalpha
    doffs = torch.empty(max(n_entries, 1), dtype=torch.float32, device=q.device) if doffs is None else doffs
    if reuse_rotated and ws is None:
        raise ValueError("reuse_rotated needs the forward's workspace")
    if ws is None:
        need = rope_frac_workspace_bytes(q.dtype, B, H, N, d, alpha=alpha, w=w, R=R, base=base)[1]
        ws = torch.empty(max(need // 4, 4), dtype=torch.int32, device=q.device)
    with torch.cuda.device(q.device):
        _check(library().fsa_rope_frac_backward(DTYPES[q.dtype], DTYPES[dq.dtype], _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(table), n_pos, _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                                _ptr(dk), _ptr(dv), _ptr(dalpha), _ptr(doffs), _ptr(ws),
                                                ws.numel() * ws.element_size(), int(bool(reuse_rotated)), B, H, N, d,
                                                _scale(scale, d), BASES[base], float(alpha), int(w), int(R),
                                                _stream(q.device)))
    return dq, dk, dv, dalpha, doffs[:n_entries]


# ----------------------------------------------------------------------------
# the one-launch backward's bounded waits
# ----------------------------------------------------------------------------


def wait_status(kind: str, q, ws, *, alpha: float = 1.0, w: int, R: int, base: str = "fib") -> bool:
    """True if the last one-launch call of `kind` ("backward", "frac_backward",
    "rope_backward", "rope_frac_backward", "backward_noalloc", or "rope_forward", the
    rotary forward that rotates K in the kernel) that ran with workspace `ws` on q's shape
    gave up one of its bounded waits (it then stored NaN results). Synchronises the
    current stream (see fsa_wait_status)."""
    B, H, N, d = q.shape
    out = ctypes.c_int32(0)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    with torch.cuda.device(q.device):
        _check(library().fsa_wait_status(WS_KINDS[kind], DTYPES[q.dtype], B, H, N, d, BASES[base], float(alpha),
                                         int(w), int(R), _ptr(ws), nbytes, ctypes.byref(out), _stream(q.device)))
    return bool(out.value)


def debug_force_wait_timeout(enable: bool) -> None:
    """Diagnostic hook: makes later one-launch waits give up (see fsa_debug_force_wait_timeout)."""
    _check(library().fsa_debug_force_wait_timeout(int(bool(enable))))


def debug_tile_order(nb: int):
    """Diagnostic hook: the logical tile each workgroup of a window-kernel grid of nb
    workgroups processes (see fsa_debug_tile_order), as a list."""
    out = (ctypes.c_int32 * max(nb, 1))()
    _check(library().fsa_debug_tile_order(int(nb), out))
    return [out[b] for b in range(nb)]
