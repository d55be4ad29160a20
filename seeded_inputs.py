"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module holds no attention arithmetic: it only draws i.i.d. standard-normal
tensors from a seeded PCG64 generator and quantises them to bfloat16 with
round-to-nearest-even on the integer bit pattern.  The GPU receives exactly the
bf16 bits produced here; the oracle receives the same values upcast to float64.

Workloads (the five problem sizes of the FlashAttention-2 backward study),
keyed by their shapes:
  n48_d16_fp32               B=1 H=1  N=48    d=16  fp32  non-causal and causal
  h8_n1024_d64_bf16          B=1 H=8  N=1024  d=64  bf16  non-causal
  h32_n8192_d128_bf16        B=1 H=32 N=8192  d=128 bf16  non-causal and causal
  b4_h16_n4000_d128_bf16_q4  B=4 H=16 N=4000  d=128 bf16  causal, Q x 4 after drawing
  h8_n32768_d128_bf16        B=1 H=8  N=32768 d=128 bf16  causal
Q, K, V, dO are drawn in that order from one generator per workload, with
seeds 0 .. 4 in the order listed; the scale is 1/sqrt(d).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp32", "bf16" or "fp16"
    causal: tuple         # causal modes this workload is run in
    seed: int
    q_mult: float = 1.0   # applied to Q after drawing (exact in bf16 for powers of two)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self, causal: bool) -> float:
        """Backward FLOP count 10*B*H*N^2*d, halved under the causal mask."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return 0.5 * f if causal else f


WORKLOADS = {w.name: w for w in (
    Workload("n48_d16_fp32", 1, 1, 48, 16, "fp32", (False, True), 0),
    Workload("h8_n1024_d64_bf16", 1, 8, 1024, 64, "bf16", (False,), 1),
    Workload("h32_n8192_d128_bf16", 1, 32, 8192, 128, "bf16", (False, True), 2),
    Workload("b4_h16_n4000_d128_bf16_q4", 4, 16, 4000, 128, "bf16", (True,), 3, q_mult=4.0),
    Workload("h8_n32768_d128_bf16", 1, 8, 32768, 128, "bf16", (True,), 4),
)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even), returned as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE half (round-to-nearest-even; beyond the largest
    half, infinity), returned as uint16 bits."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of IEEE half bit patterns to float32."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


@dataclass
class Inputs:
    """Q, K, V, dO as float32 arrays holding exactly representable values.

    For bf16 and fp16 workloads ``bits`` holds the uint16 patterns that go to
    the GPU and the float32 arrays are their exact widening.
    """
    wl: Workload
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    dO: np.ndarray
    bits: dict = field(default_factory=dict)


def draw(wl: Workload, *, B=None, H=None, N=None, d=None, seed=None, q_mult=None,
         dtype=None) -> Inputs:
    """Draw Q, K, V, dO of shape [B,H,N,d] for a workload (fields overridable)."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    N = wl.N if N is None else N
    d = wl.d if d is None else d
    seed = wl.seed if seed is None else seed
    q_mult = wl.q_mult if q_mult is None else q_mult
    dtype = wl.dtype if dtype is None else dtype
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    arrs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(4)]
    if q_mult != 1.0:
        arrs[0] = arrs[0] * np.float32(q_mult)
    names = ("Q", "K", "V", "dO")
    wl2 = Workload(wl.name, B, H, N, d, dtype, wl.causal, seed, q_mult)
    if dtype == "bf16":
        bits = {n: f32_to_bf16_bits(a) for n, a in zip(names, arrs)}
        vals = [bf16_bits_to_f32(bits[n]) for n in names]
        return Inputs(wl2, *vals, bits=bits)
    if dtype == "fp16":
        bits = {n: f32_to_f16_bits(a) for n, a in zip(names, arrs)}
        vals = [f16_bits_to_f32(bits[n]) for n in names]
        return Inputs(wl2, *vals, bits=bits)
    if dtype == "fp32":
        return Inputs(wl2, *arrs)
    raise ValueError(f"unknown dtype {dtype}")


def draw_custom(B, H, N, d, dtype, seed, q_mult=1.0) -> Inputs:
    """Draw inputs for an arbitrary shape (edge-case tests)."""
    wl = Workload("custom", B, H, N, d, dtype, (False, True), seed, q_mult)
    return draw(wl)
