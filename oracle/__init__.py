"""CPU fp64 oracle for attention forward and backward (ctypes over attn_oracle.c).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library and never imports it.

The functions follow the chain rule of the FlashAttention-2 backward as the
pages state it (see the header of attn_oracle.c for the citations):
``attn_fwd``/``attn_bwd`` are the plain definitions, ``row_stats``,
``fwd_rows``, ``dq_rows`` and ``dkdv_rows`` compute selected outputs of the same
definitions for problems too large to do whole, and ``flash_fwd_tiled`` /
``flash_bwd_tiled`` are the tiled online-softmax / key-outer variants used only
to check the definitions.

All arrays are float64, contiguous, shaped [B, H, N, d] (L and D: [B, H, N]).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

FLAG_FORGET_ALPHA_ON_ACC = 1


def build() -> str:
    """Compile attn_oracle.c with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.POINTER(ctypes.c_double)
    PL = ctypes.POINTER(ctypes.c_long)
    l, dbl, i = ctypes.c_long, ctypes.c_double, ctypes.c_int
    sig = {
        "orc_attn_fwd": [P, P, P, l, l, l, dbl, i, P, P],
        "orc_attn_bwd": [P, P, P, P, l, l, l, dbl, i, P, P, P, P],
        "orc_row_stats": [P, P, P, P, l, l, dbl, i, P, P],
        "orc_fwd_rows": [P, P, P, l, l, dbl, i, PL, l, P, P],
        "orc_dq_rows": [P, P, P, P, l, l, dbl, i, PL, l, P],
        "orc_dkdv_rows": [P, P, P, P, P, P, l, l, dbl, i, PL, l, P, P],
        "orc_flash_fwd_tiled": [P, P, P, l, l, l, dbl, i, l, l, i, P, P],
        "orc_flash_bwd_tiled": [P, P, P, P, P, P, l, l, l, dbl, i, l, l, P, P, P],
        "orc_set_threads": [i],
        "orc_max_threads": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int if name == "orc_max_threads" else None
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _idx(rows) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def max_threads() -> int:
    return _load().orc_max_threads()


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def attn_fwd(Q, K, V, scale, causal):
    """O, L of standard attention (softmax over scaled, masked scores)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    *lead, N, d = Q.shape
    BH = int(np.prod(lead)) if lead else 1
    O = np.empty_like(Q)
    L = np.empty(tuple(lead) + (N,), dtype=np.float64)
    _load().orc_attn_fwd(_p(Q), _p(K), _p(V), BH, N, d, float(scale), int(causal), _p(O), _p(L))
    return O, L


def attn_bwd(Q, K, V, dO, scale, causal):
    """dQ, dK, dV (and D) of standard attention by the chain rule."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    *lead, N, d = Q.shape
    BH = int(np.prod(lead)) if lead else 1
    dQ, dK, dV = np.empty_like(Q), np.empty_like(Q), np.empty_like(Q)
    D = np.empty(tuple(lead) + (N,), dtype=np.float64)
    _load().orc_attn_bwd(_p(Q), _p(K), _p(V), _p(dO), BH, N, d, float(scale), int(causal),
                         _p(dQ), _p(dK), _p(dV), _p(D))
    return dQ, dK, dV, D


def row_stats(Q, K, V, dO, scale, causal):
    """L_i and D_i (by definition) for every row of ONE head ([N, d] inputs)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    N, d = Q.shape
    L = np.empty(N)
    D = np.empty(N)
    _load().orc_row_stats(_p(Q), _p(K), _p(V), _p(dO), N, d, float(scale), int(causal), _p(L), _p(D))
    return L, D


def fwd_rows(Q, K, V, scale, causal, rows):
    """O and L of selected rows of ONE head."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    N, d = Q.shape
    r = _idx(rows)
    O = np.empty((len(r), d))
    L = np.empty(len(r))
    _load().orc_fwd_rows(_p(Q), _p(K), _p(V), N, d, float(scale), int(causal),
                         r.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), len(r), _p(O), _p(L))
    return O, L


def dq_rows(Q, K, V, dO, scale, causal, rows):
    """dQ of selected rows of ONE head."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    N, d = Q.shape
    r = _idx(rows)
    out = np.empty((len(r), d))
    _load().orc_dq_rows(_p(Q), _p(K), _p(V), _p(dO), N, d, float(scale), int(causal),
                        r.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), len(r), _p(out))
    return out


def dkdv_rows(Q, K, V, dO, L, D, scale, causal, keys):
    """dK and dV of selected keys of ONE head, given that head's L and D."""
    Q, K, V, dO, L, D = _f64(Q), _f64(K), _f64(V), _f64(dO), _f64(L), _f64(D)
    N, d = Q.shape
    r = _idx(keys)
    dk = np.empty((len(r), d))
    dv = np.empty((len(r), d))
    _load().orc_dkdv_rows(_p(Q), _p(K), _p(V), _p(dO), _p(L), _p(D), N, d, float(scale),
                          int(causal), r.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), len(r),
                          _p(dk), _p(dv))
    return dk, dv


def flash_fwd_tiled(Q, K, V, scale, causal, Br, Bc, flags=0):
    """Tiled online-softmax forward (check of attn_fwd)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    *lead, N, d = Q.shape
    BH = int(np.prod(lead)) if lead else 1
    O = np.empty_like(Q)
    L = np.empty(tuple(lead) + (N,), dtype=np.float64)
    _load().orc_flash_fwd_tiled(_p(Q), _p(K), _p(V), BH, N, d, float(scale), int(causal),
                                int(Br), int(Bc), int(flags), _p(O), _p(L))
    return O, L


def flash_bwd_tiled(Q, K, V, O, dO, L, scale, causal, Br, Bc):
    """Key-outer / query-inner tiled backward from O and L (check of attn_bwd)."""
    Q, K, V, O, dO, L = _f64(Q), _f64(K), _f64(V), _f64(O), _f64(dO), _f64(L)
    *lead, N, d = Q.shape
    BH = int(np.prod(lead)) if lead else 1
    dQ, dK, dV = np.empty_like(Q), np.empty_like(Q), np.empty_like(Q)
    _load().orc_flash_bwd_tiled(_p(Q), _p(K), _p(V), _p(O), _p(dO), _p(L), BH, N, d,
                                float(scale), int(causal), int(Br), int(Bc),
                                _p(dQ), _p(dK), _p(dV))
    return dQ, dK, dV
