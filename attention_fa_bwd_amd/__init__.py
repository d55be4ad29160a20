"""MI355X (gfx950) FlashAttention-2 backward: thin ctypes binding over libfa_bwd.so.

The entry points mirror include/fa_bwd.h one for one (argument marshalling
only: every step runs in the HIP kernels of the library).  PyTorch provides
device memory and the current stream.  There is no fallback: if the library is
missing or returns an error, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FA_DTYPE_F32", "FA_DTYPE_BF16", "FA_DTYPE_F16", "FAError", "lib_path", "load",
    "fa_fwd_lse", "fa_lse", "fa_bwd_preprocess", "fa_bwd", "fa_bwd_dkdv", "fa_bwd_dq",
    "fa_bwd_convert_dq", "fa_bwd_noalloc", "fa_strerror",
    "forward", "lse", "backward",
]

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2
FA_OK, FA_EINVAL, FA_EUNSUPPORTED, FA_EHIP, FA_ESCRATCH = 0, 1, 2, 3, 4
FA_NOALLOC_MAX_ROWS = 1 << 22   # B * H * N rows that fa_bwd_noalloc's scratch holds

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa_bwd.so")
_lib = None

# name -> argtypes (void* for pointers, stream last); every function returns int
_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_SIGS = {
    "fa_fwd_lse": [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_lse": [_i, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_preprocess": [_i, _vp, _vp, _vp, _i, _i, _i, _i, _vp],
    "fa_bwd": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_dkdv": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_dq": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_convert_dq": [_i, _vp, _vp, _i, _i, _i, _i, _f, _vp],
    "fa_bwd_noalloc": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_last_hip_error": [],
}


class FAError(RuntimeError):
    def __init__(self, fn, status, hip_err=0):
        self.status, self.hip_error = status, hip_err
        msg = f"{fn}: {fa_strerror(status)}"
        if status == FA_EHIP:
            msg += f" (hipError_t {hip_err})"
        super().__init__(msg)


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libfa_bwd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m attention_fa_bwd_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.fa_strerror.argtypes = [_i]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: torch.Tensor, dtype=None, ref=None) -> int:
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if ref is not None and t.device != ref.device:
        raise ValueError(f"tensors on different devices: {t.device} and {ref.device}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _ptrs(ref, *specs):
    """Device addresses for (tensor, dtype, shape) triples, after the checks the
    C-ABI cannot make: first every shape against the one the call's sizes
    imply (a smaller buffer would be read or written out of bounds), then
    device (that of ``ref``), contiguity and element type."""
    for t, _, shape in specs:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return [_ptr(t, dtype, ref) for t, dtype, _ in specs]


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, rc: int):
    if rc != FA_OK:
        raise FAError(fn, rc, load().fa_last_hip_error())


def _shape(t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    return tuple(int(x) for x in t.shape)


def _sizes(t):
    B, H, N, d = _shape(t)
    return (B, H, N, d), (B, H, N)


def fa_fwd_lse(q, k, v, o, L, scale: float, causal: bool, stream=None) -> None:
    s4, s3 = _sizes(q)
    e = q.dtype
    ptrs = _ptrs(q, (q, e, s4), (k, e, s4), (v, e, s4), (o, e, s4), (L, torch.float32, s3))
    rc = load().fa_fwd_lse(_dtype_code(q), *ptrs, *s4, float(scale), int(bool(causal)),
                           _stream(stream))
    _check("fa_fwd_lse", rc)


def fa_lse(q, k, L, scale: float, causal: bool, stream=None) -> None:
    s4, s3 = _sizes(q)
    ptrs = _ptrs(q, (q, q.dtype, s4), (k, q.dtype, s4), (L, torch.float32, s3))
    rc = load().fa_lse(_dtype_code(q), *ptrs, *s4, float(scale), int(bool(causal)),
                       _stream(stream))
    _check("fa_lse", rc)


def fa_bwd_preprocess(o, do, D, stream=None) -> None:
    s4, s3 = _sizes(o)
    ptrs = _ptrs(o, (o, o.dtype, s4), (do, o.dtype, s4), (D, torch.float32, s3))
    rc = load().fa_bwd_preprocess(_dtype_code(o), *ptrs, *s4, _stream(stream))
    _check("fa_bwd_preprocess", rc)


def _bwd_inputs(q, k, v, do, L, D):
    s4, s3 = _sizes(q)
    e, f = q.dtype, torch.float32
    return [(q, e, s4), (k, e, s4), (v, e, s4), (do, e, s4), (L, f, s3), (D, f, s3)]


def fa_bwd(q, k, v, do, L, D, dq_accum, dk, dv, scale: float, causal: bool, stream=None) -> None:
    s4, _ = _sizes(q)
    ptrs = _ptrs(q, *_bwd_inputs(q, k, v, do, L, D), (dq_accum, torch.float32, s4),
                 (dk, q.dtype, s4), (dv, q.dtype, s4))
    rc = load().fa_bwd(_dtype_code(q), *ptrs, *s4, float(scale), int(bool(causal)),
                       _stream(stream))
    _check("fa_bwd", rc)


def fa_bwd_dkdv(q, k, v, do, L, D, dk, dv, scale: float, causal: bool, stream=None) -> None:
    s4, _ = _sizes(q)
    ptrs = _ptrs(q, *_bwd_inputs(q, k, v, do, L, D), (dk, q.dtype, s4), (dv, q.dtype, s4))
    rc = load().fa_bwd_dkdv(_dtype_code(q), *ptrs, *s4, float(scale), int(bool(causal)),
                            _stream(stream))
    _check("fa_bwd_dkdv", rc)


def fa_bwd_dq(q, k, v, do, L, D, dq_accum, scale: float, causal: bool, stream=None) -> None:
    s4, _ = _sizes(q)
    ptrs = _ptrs(q, *_bwd_inputs(q, k, v, do, L, D), (dq_accum, torch.float32, s4))
    rc = load().fa_bwd_dq(_dtype_code(q), *ptrs, *s4, float(scale), int(bool(causal)),
                          _stream(stream))
    _check("fa_bwd_dq", rc)


def fa_bwd_convert_dq(dq_accum, dq, scale: float, stream=None) -> None:
    s4, _ = _sizes(dq)
    ptrs = _ptrs(dq, (dq_accum, torch.float32, s4), (dq, dq.dtype, s4))
    rc = load().fa_bwd_convert_dq(_dtype_code(dq), *ptrs, *s4, float(scale), _stream(stream))
    _check("fa_bwd_convert_dq", rc)


def fa_bwd_noalloc(q, k, v, o, do, L, dq, dk, dv, scale: float, causal: bool,
                   stream=None) -> None:
    """The whole backward with no device allocation (D in the library's static
    scratch, dQ written scaled by the dQ pass)."""
    s4, s3 = _sizes(q)
    e = q.dtype
    ptrs = _ptrs(q, (q, e, s4), (k, e, s4), (v, e, s4), (o, e, s4), (do, e, s4),
                 (L, torch.float32, s3), (dq, e, s4), (dk, e, s4), (dv, e, s4))
    rc = load().fa_bwd_noalloc(_dtype_code(q), *ptrs, *s4, float(scale), int(bool(causal)),
                               _stream(stream))
    _check("fa_bwd_noalloc", rc)


def forward(q, k, v, scale: float, causal: bool, stream=None):
    """O and L for the given inputs (allocates both)."""
    B, H, N, d = _shape(q)
    o = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_lse(q, k, v, o, L, scale, causal, stream)
    return o, L


def lse(q, k, scale: float, causal: bool, stream=None):
    """L alone (allocates it): for a backward whose forward did not keep L."""
    B, H, N, d = _shape(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_lse(q, k, L, scale, causal, stream)
    return L


def backward(q, k, v, o, do, L, scale: float, causal: bool, stream=None, workspace=None):
    """dQ, dK, dV: preprocess, main kernel and convert, in order on one stream.

    ``workspace`` may hold preallocated (D, dq_accum) buffers."""
    B, H, N, d = _shape(q)
    if workspace is None:
        D = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        dq_accum = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    else:
        D, dq_accum = workspace
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    fa_bwd_preprocess(o, do, D, stream)
    fa_bwd(q, k, v, do, L, D, dq_accum, dk, dv, scale, causal, stream)
    fa_bwd_convert_dq(dq_accum, dq, scale, stream)
    return dq, dk, dv
