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
    "fa_bwd_convert_dq", "fa_strerror",
    "forward", "lse", "backward",
]

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2
FA_OK, FA_EINVAL, FA_EUNSUPPORTED, FA_EHIP = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa_bwd.so")
_lib = None

# name -> argtypes (void* for pointers, stream last); every function returns int
_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_SIGS = {
    "fa_fwd_lse": [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_lse": [_i, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_preprocess": [_i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp],
    "fa_bwd": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_dkdv": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_dq": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp],
    "fa_bwd_convert_dq": [_i, _vp, _vp, _i, _i, _i, _i, _f, _vp],
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


def _ptr(t: torch.Tensor, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


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


def fa_fwd_lse(q, k, v, o, L, scale: float, causal: bool, stream=None) -> None:
    B, H, N, d = _shape(q)
    dt = _dtype_code(q)
    rc = load().fa_fwd_lse(dt, _ptr(q, q.dtype), _ptr(k, q.dtype), _ptr(v, q.dtype),
                           _ptr(o, q.dtype), _ptr(L, torch.float32), B, H, N, d,
                           float(scale), int(bool(causal)), _stream(stream))
    _check("fa_fwd_lse", rc)


def fa_lse(q, k, L, scale: float, causal: bool, stream=None) -> None:
    B, H, N, d = _shape(q)
    dt = _dtype_code(q)
    rc = load().fa_lse(dt, _ptr(q, q.dtype), _ptr(k, q.dtype), _ptr(L, torch.float32),
                       B, H, N, d, float(scale), int(bool(causal)), _stream(stream))
    _check("fa_lse", rc)


def fa_bwd_preprocess(o, do, D, dq_accum, stream=None) -> None:
    B, H, N, d = _shape(o)
    dt = _dtype_code(o)
    rc = load().fa_bwd_preprocess(dt, _ptr(o, o.dtype), _ptr(do, o.dtype),
                                  _ptr(D, torch.float32), _ptr(dq_accum, torch.float32),
                                  B, H, N, d, _stream(stream))
    _check("fa_bwd_preprocess", rc)


def fa_bwd(q, k, v, do, L, D, dq_accum, dk, dv, scale: float, causal: bool, stream=None) -> None:
    B, H, N, d = _shape(q)
    dt = _dtype_code(q)
    rc = load().fa_bwd(dt, _ptr(q, q.dtype), _ptr(k, q.dtype), _ptr(v, q.dtype),
                       _ptr(do, q.dtype), _ptr(L, torch.float32), _ptr(D, torch.float32),
                       _ptr(dq_accum, torch.float32), _ptr(dk, q.dtype), _ptr(dv, q.dtype),
                       B, H, N, d, float(scale), int(bool(causal)), _stream(stream))
    _check("fa_bwd", rc)


def fa_bwd_dkdv(q, k, v, do, L, D, dk, dv, scale: float, causal: bool, stream=None) -> None:
    B, H, N, d = _shape(q)
    dt = _dtype_code(q)
    rc = load().fa_bwd_dkdv(dt, _ptr(q, q.dtype), _ptr(k, q.dtype), _ptr(v, q.dtype),
                            _ptr(do, q.dtype), _ptr(L, torch.float32), _ptr(D, torch.float32),
                            _ptr(dk, q.dtype), _ptr(dv, q.dtype), B, H, N, d, float(scale),
                            int(bool(causal)), _stream(stream))
    _check("fa_bwd_dkdv", rc)


def fa_bwd_dq(q, k, v, do, L, D, dq_accum, scale: float, causal: bool, stream=None) -> None:
    B, H, N, d = _shape(q)
    dt = _dtype_code(q)
    rc = load().fa_bwd_dq(dt, _ptr(q, q.dtype), _ptr(k, q.dtype), _ptr(v, q.dtype),
                          _ptr(do, q.dtype), _ptr(L, torch.float32), _ptr(D, torch.float32),
                          _ptr(dq_accum, torch.float32), B, H, N, d, float(scale),
                          int(bool(causal)), _stream(stream))
    _check("fa_bwd_dq", rc)


def fa_bwd_convert_dq(dq_accum, dq, scale: float, stream=None) -> None:
    B, H, N, d = _shape(dq)
    dt = _dtype_code(dq)
    rc = load().fa_bwd_convert_dq(dt, _ptr(dq_accum, torch.float32), _ptr(dq, dq.dtype),
                                  B, H, N, d, float(scale), _stream(stream))
    _check("fa_bwd_convert_dq", rc)


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
    fa_bwd_preprocess(o, do, D, dq_accum, stream)
    fa_bwd(q, k, v, do, L, D, dq_accum, dk, dv, scale, causal, stream)
    fa_bwd_convert_dq(dq_accum, dq, scale, stream)
    return dq, dk, dv
