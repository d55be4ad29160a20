"""GPU parity of the forward (fa_fwd_lse) and of L alone (fa_lse): O and L
against the oracle's plain definition, element by element.

bf16 and fp16 with d = 64 or 128 run the matrix-core kernel (lazy rebase of the
running maximum); the other cases run the vector-ALU kernel.  Tolerances: O within the
element type's bar (max |err| / max |ref|), L (natural log, fp32) within 1e-4
absolute -- S comes from exact 16-bit products accumulated in fp32, so L is
accurate to a few fp32 ulps of the scores."""
import numpy as np
import torch
import pytest

import gpu_util as gu
import oracle
import seeded_inputs as si
import attention_fa_bwd_amd as fa

pytestmark = pytest.mark.gpu


def _forward(inp, causal):
    q, k, v = (gu.upload(inp, n) for n in ("Q", "K", "V"))
    o, L = fa.forward(q, k, v, inp.wl.scale, causal)
    return gu.to_f64(o), gu.to_f64(L)


def _check(inp, causal, what, l_tol=1e-4):
    o, L = _forward(inp, causal)
    O, Lr = oracle.attn_fwd(inp.Q, inp.K, inp.V, inp.wl.scale, causal)
    eo = gu.rel_err(o, O)
    el = float(np.abs(L - Lr).max())
    gu.note(f"  {what}: o {eo:.3e}  L {el:.3e}")
    assert not np.isnan(o).any() and not np.isnan(L).any()
    assert eo <= gu.TOL[inp.wl.dtype], f"{what}: O rel err {eo:.3e}"
    assert el <= l_tol, f"{what}: L abs err {el:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 200, 255, 256, 257, 600])
def test_matrix_core_shapes(N, causal, dtype, d):
    """Matrix-core forward: tiny, ragged and multi-block N (the workgroup holds
    256 queries, key blocks are 64 rows)."""
    gu.note(f"case fwd {dtype} d={d} N={N} causal={causal}")
    inp = si.draw_custom(2, 2, N, d, dtype, seed=300 + N + d)
    _check(inp, causal, f"N={N} d={d}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", [(16, "fp32"), (32, "bf16"), (16, "fp16"), (128, "fp32")])
def test_vector_alu_forward(d, dtype, causal):
    gu.note(f"case fwd {dtype} d={d} causal={causal}")
    inp = si.draw_custom(1, 2, 133, d, dtype, seed=400 + d)
    _check(inp, causal, f"{dtype} d={d}", l_tol=1e-6 if dtype == "fp32" else 1e-4)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("q_mult", [4.0, 8.0])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_large_scores(q_mult, causal, d):
    """Peaky softmax: row maxima of tens to hundreds in exp2 units, so the
    running maximum moves by more than the lazy threshold many times."""
    gu.note(f"case fwd large scores d={d} q x{q_mult} causal={causal}")
    inp = si.draw_custom(1, 2, 700, d, "bf16", seed=500 + int(q_mult), q_mult=q_mult)
    _check(inp, causal, f"q x{q_mult}", l_tol=1e-3)


def test_bf16_d128_growing_max():
    """Scores grow along the keys (K rows scaled up with their index), so
    nearly every key block carries a new row maximum: the rebase path runs in
    most blocks, for every query."""
    gu.note("case fwd growing max")
    inp = si.draw_custom(1, 1, 1024, 128, "bf16", seed=77)
    N = inp.wl.N
    grow = (1.0 + 6.0 * np.arange(N, dtype=np.float32) / N)[None, None, :, None]
    bits = si.f32_to_bf16_bits(inp.K * grow)
    inp.bits["K"] = bits
    inp.K = si.bf16_bits_to_f32(bits)
    _check(inp, False, "growing max", l_tol=1e-3)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 128), ("bf16", 64), ("fp16", 64), ("fp16", 32),
                                     ("fp32", 16), ("fp32", 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 257, 600])
def test_lse_alone(N, causal, dtype, d):
    """fa_lse (L without O, for a backward whose forward did not keep L):
    against the oracle's plain definition, and bitwise equal to the forward's
    L on the same inputs -- the same sweep with V left out."""
    gu.note(f"case lse {dtype} d={d} N={N} causal={causal}")
    inp = si.draw_custom(2, 2, N, d, dtype, seed=600 + N + d)
    q, k, v = (gu.upload(inp, n) for n in ("Q", "K", "V"))
    L = fa.lse(q, k, inp.wl.scale, causal)
    _, Lf = fa.forward(q, k, v, inp.wl.scale, causal)
    assert torch.equal(L, Lf)
    _, Lr = oracle.attn_fwd(inp.Q, inp.K, inp.V, inp.wl.scale, causal)
    el = float(np.abs(gu.to_f64(L) - Lr).max())
    gu.note(f"  L {el:.3e}")
    # fp32: the score dot products and the running sum each add a few
    # roundings, so L is good to a few ulps of its own magnitude
    bar = 8 * 2.0**-23 * max(1.0, float(np.abs(Lr).max())) if dtype == "fp32" else 1e-4
    assert el <= bar, f"L abs err {el:.3e} > {bar:.3e}"


@pytest.mark.parametrize("causal", [False, True])
def test_lse_alone_large_scores(causal):
    """Peaky rows: the running maximum moves past the lazy threshold often."""
    gu.note(f"case lse large scores causal={causal}")
    inp = si.draw_custom(1, 2, 700, 128, "bf16", seed=508, q_mult=8.0)
    q, k = gu.upload(inp, "Q"), gu.upload(inp, "K")
    L = fa.lse(q, k, inp.wl.scale, causal)
    _, Lr = oracle.attn_fwd(inp.Q, inp.K, inp.V, inp.wl.scale, causal)
    el = float(np.abs(gu.to_f64(L) - Lr).max())
    assert el <= 1e-3, f"L abs err {el:.3e}"
