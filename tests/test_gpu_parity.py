"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle on
the same seeded inputs.

Bar (per gradient tensor): max|g_gpu - g_ref| / max|g_ref| <= 1e-5 for fp32
and <= 2e-2 for bf16.  Small problems are compared element by element over
whole tensors; the full-size workloads are compared on sampled rows of sampled
heads (the oracle computes those one by one) and through invariants that hold
at any size.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_util as gu
else:  # collected on CPU-only machines, never run there
    gu = None


def _assert_grads(errs, tol, what):
    for n in ("dq", "dk", "dv"):
        assert errs[n] <= tol, f"{what}: {n} rel err {errs[n]:.3e} > {tol}"


# ---------------------------------------------------------------- workload n48_d16_fp32

@pytest.mark.parametrize("causal", [False, True])
def test_c1_fp32_oracle_O_L(causal):
    """N=48, d=16, fp32: O and L from the oracle forward feed the GPU backward."""
    wl = si.WORKLOADS["n48_d16_fp32"]
    gu.note(f"case n48_d16_fp32 fp32 causal={causal} (oracle O, L)")
    inp = si.draw(wl)
    O, L = oracle.attn_fwd(inp.Q, inp.K, inp.V, wl.scale, causal)
    out = gu.run_gpu(inp, causal, O=O.astype(np.float32), L=L)
    errs = gu.compare_full(inp, causal, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL["fp32"], "n48_d16_fp32")
    assert errs["D"] <= 1e-5


@pytest.mark.parametrize("causal", [False, True])
def test_c1_fp32_end_to_end(causal):
    wl = si.WORKLOADS["n48_d16_fp32"]
    gu.note(f"case n48_d16_fp32 fp32 causal={causal} (GPU forward)")
    inp = si.draw(wl)
    out = gu.run_gpu(inp, causal)
    errs = gu.compare_full(inp, causal, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL["fp32"], "n48_d16_fp32 e2e")
    assert errs["o"] <= 1e-5 and errs["L"] <= 1e-5


# ---------------------------------------------------------------- workload h8_n1024_d64_bf16

@pytest.mark.parametrize("causal", [False, True])
def test_c2_bf16_full(causal):
    """B=1, H=8, N=1024, d=64 bf16 (the workload is non-causal; causal added)."""
    wl = si.WORKLOADS["h8_n1024_d64_bf16"]
    gu.note(f"case h8_n1024_d64_bf16 bf16 causal={causal}")
    inp = si.draw(wl)
    out = gu.run_gpu(inp, causal)
    errs = gu.compare_full(inp, causal, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL["bf16"], "h8_n1024_d64_bf16")
    assert errs["o"] <= 2e-2 and errs["L"] <= 1e-3


def test_c2_isolated_backward():
    """The oracle's O (rounded to bf16) and L feed the GPU backward."""
    wl = si.WORKLOADS["h8_n1024_d64_bf16"]
    gu.note("case h8_n1024_d64_bf16 bf16 isolated backward")
    inp = si.draw(wl)
    O, L = oracle.attn_fwd(inp.Q, inp.K, inp.V, wl.scale, False)
    out = gu.run_gpu(inp, False, O=O.astype(np.float32), L=L)
    errs = gu.compare_full(inp, False, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL["bf16"], "h8_n1024_d64_bf16 isolated")


# ------------------------------------------------------------ edge shapes

EDGE_N = [1, 2, 17, 47, 63, 64, 65, 127, 129, 200]
EDGE_D = [(d, dt) for d in (16, 32, 64, 128) for dt in ("bf16", "fp32")] + [(64, "fp16"), (128, "fp16")]


def _stored(O, dtype):
    """The forward output as the method stores it (16-bit types: round to
    nearest even)."""
    if dtype == "bf16":
        return si.bf16_bits_to_f32(si.f32_to_bf16_bits(O.astype(np.float32)))
    if dtype == "fp16":
        return si.f16_bits_to_f32(si.f32_to_f16_bits(O.astype(np.float32)))
    return O.astype(np.float32)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", EDGE_D, ids=[f"{dt}-d{d}" for d, dt in EDGE_D])
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_shapes(N, d, dtype, causal):
    """Ragged and tiny N for every head dim and dtype.

    (1) Isolated backward: the oracle's O, stored in the element type, and its L
        feed the GPU backward; the reference is the oracle's key-outer backward
        consuming the same stored O (D = dO . O).
    (2) End to end (GPU forward, then backward) against the plain definition,
        for N >= 16.  Below that, D formed from a bf16-stored O can dominate:
        with two keys dS is a small difference (N=2 emulated on the CPU gives
        2.2e-2 on dK), so the chain is checked link by link instead: the GPU
        forward's O and L against the oracle's forward, then the GPU backward
        that consumed them against the oracle's key-outer backward fed the
        very same stored O and L."""
    gu.note(f"case edge N={N} d={d} {dtype} causal={causal}")
    inp = si.draw_custom(1, 2, N, d, dtype, seed=100 + N + d)
    scale = inp.wl.scale
    O, L = oracle.attn_fwd(inp.Q, inp.K, inp.V, scale, causal)
    Os = _stored(O, dtype)
    out = gu.run_gpu(inp, causal, O=Os, L=L)
    rq, rk, rv = oracle.flash_bwd_tiled(inp.Q, inp.K, inp.V, Os, inp.dO, L, scale, causal, 16, 12)
    errs = {n: gu.rel_err(gu.to_f64(out[n]), r) for n, r in (("dq", rq), ("dk", rk), ("dv", rv))}
    _assert_grads(errs, gu.TOL[dtype], f"isolated N={N} d={d} {dtype}")
    assert not gu.invariants(inp, causal, out)["nan"]
    out = gu.run_gpu(inp, causal)
    if N >= 16 or dtype == "fp32":
        errs = gu.compare_full(inp, causal, out)
        _assert_grads(errs, gu.TOL[dtype], f"N={N} d={d} {dtype}")
    else:
        eo = gu.rel_err(gu.to_f64(out["o"]), O)
        el = float(np.abs(gu.to_f64(out["L"]) - L).max())
        assert eo <= gu.TOL[dtype] and el <= 1e-4, f"forward N={N}: O {eo:.3e}, L {el:.3e}"
        Og, Lg = gu.to_f64(out["o"]), gu.to_f64(out["L"])
        rq, rk, rv = oracle.flash_bwd_tiled(inp.Q, inp.K, inp.V, Og, inp.dO, Lg, scale, causal, 16, 12)
        errs = {n: gu.rel_err(gu.to_f64(out[n]), r) for n, r in (("dq", rq), ("dk", rk), ("dv", rv))}
        _assert_grads(errs, gu.TOL[dtype], f"chained N={N} d={d} {dtype}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [300, 520])
def test_multi_block_ragged(N, d, dtype, causal):
    """Matrix-core head dims: more than one 256-query block of the dQ pass and
    more than one 128-key block of the dK/dV pass, the last of each ragged
    (N = 300: 44 rows in the second query block, so three of its four score
    waves own only rows past N; N = 520: 8 rows in the third).  Full tensors
    against the oracle, end to end and with the oracle's O and L."""
    gu.note(f"case multi-block ragged N={N} d={d} {dtype} causal={causal}")
    inp = si.draw_custom(2, 2, N, d, dtype, seed=900 + N + d)
    out = gu.run_gpu(inp, causal)
    errs = gu.compare_full(inp, causal, out)
    _assert_grads(errs, gu.TOL[dtype], f"N={N} d={d} {dtype} end to end")
    O, L = oracle.attn_fwd(inp.Q, inp.K, inp.V, inp.wl.scale, causal)
    Os = _stored(O, dtype)
    out = gu.run_gpu(inp, causal, O=Os, L=L)
    rq, rk, rv = oracle.flash_bwd_tiled(inp.Q, inp.K, inp.V, Os, inp.dO, L, inp.wl.scale, causal, 16, 12)
    errs = {n: gu.rel_err(gu.to_f64(out[n]), r) for n, r in (("dq", rq), ("dk", rk), ("dv", rv))}
    _assert_grads(errs, gu.TOL[dtype], f"N={N} d={d} {dtype} isolated")
    assert not gu.invariants(inp, causal, out)["nan"]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_xcd_order_and_head_pairs(d, causal):
    """B=1 H=16 N=1024: every pass has a work-item count divisible by the 8 XCDs
    (dK/dV 8 key blocks x 16 heads, dQ and forward 4 query blocks x 16 heads),
    so the XCD-contiguous order is on, and under the causal mask each XCD's
    share holds whole head pairs, so the heavy-first pair interleave is on
    too.  Whole tensors against the oracle."""
    gu.note(f"case xcd order / head pairs d={d} causal={causal}")
    inp = si.draw_custom(1, 16, 1024, d, "bf16", seed=1200 + d)
    out = gu.run_gpu(inp, causal)
    errs = gu.compare_full(inp, causal, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL["bf16"], f"H=16 N=1024 d={d}")
    assert errs["o"] <= gu.TOL["bf16"] and errs["L"] <= 1e-3


MANY = [(2, 96), (1, 91)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H", MANY, ids=[f"B{b}H{h}" for b, h in MANY])
def test_many_items_per_workgroup(B, H, d, causal):
    """More work items than CUs, so every workgroup of the persistent grids
    runs several items back to back (the next item's first tiles overlap the
    previous item's last ones), at a ragged N = 300: B=2 H=96 gives item counts
    divisible by 8 (dK/dV 576, dQ 384: the XCD shares and snake order are on),
    B=1 H=91 counts that are not (273, 182: one share over all workgroups).
    Whole tensors against the oracle; the split passes and the no-allocation
    entry point bitwise equal to fa_bwd's results on the same shape."""
    import attention_fa_bwd_amd as fa
    gu.note(f"case many items per workgroup B={B} H={H} N=300 d={d} causal={causal}")
    inp = si.draw_custom(B, H, 300, d, "bf16", seed=1500 + H + d)
    out = gu.run_gpu(inp, causal)
    errs = gu.compare_full(inp, causal, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL["bf16"], f"B={B} H={H} d={d}")
    assert errs["o"] <= gu.TOL["bf16"] and errs["L"] <= 1e-3
    q, k, v, do, L, D = (out[n] for n in ("q", "k", "v", "do", "L", "D"))
    dqa = torch.full_like(out["dq_accum"], float("nan"))
    dk, dv = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
    fa.fa_bwd_dq(q, k, v, do, L, D, dqa, inp.wl.scale, causal)
    fa.fa_bwd_dkdv(q, k, v, do, L, D, dk, dv, inp.wl.scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(dqa, out["dq_accum"])
    assert torch.equal(dk, out["dk"]) and torch.equal(dv, out["dv"])
    dq2, dk2, dv2 = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.fa_bwd_noalloc(q, k, v, out["o"], do, L, dq2, dk2, dv2, inp.wl.scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(dq2, out["dq"])
    assert torch.equal(dk2, out["dk"]) and torch.equal(dv2, out["dv"])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("q_mult", [4.0, 8.0])
@pytest.mark.parametrize("causal", [False, True])
def test_large_scores(q_mult, causal, dtype, d):
    """Peaky softmax: Q scaled up so row maxima are large and land anywhere."""
    gu.note(f"case large scores d={d} q x{q_mult} causal={causal} {dtype}")
    inp = si.draw_custom(2, 2, 300, d, dtype, seed=17, q_mult=q_mult)
    out = gu.run_gpu(inp, causal)
    errs = gu.compare_full(inp, causal, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL[dtype], "large scores")


def test_max_in_last_key_block():
    """Every row's maximum score sits in the last key block (keys there are
    parallel to the queries), so the forward's running max keeps moving."""
    gu.note("case max in last key block")
    inp = si.draw_custom(1, 1, 256, 64, "fp32", seed=23)
    inp.K[0, 0, -64:] = inp.Q[0, 0, -64:] * 2.0
    out = gu.run_gpu(inp, False)
    errs = gu.compare_full(inp, False, out)
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL["fp32"], "max in last block")
    assert errs["o"] <= 1e-5


REPEAT = [(d, dt) for d in (16, 32, 64, 128) for dt in ("fp32", "bf16", "fp16")]


@pytest.mark.parametrize("d,dtype", REPEAT, ids=[f"{dt}-d{d}" for d, dt in REPEAT])
def test_bitwise_repeatable(d, dtype):
    """No path uses atomics: dq_accum, dQ, dK and dV are bitwise the same from
    one call to the next, for every dtype and head dim."""
    gu.note(f"case repeatability d={d} {dtype}")
    inp = si.draw_custom(1, 4, 300, d, dtype, seed=1)
    a = gu.run_gpu(inp, True)
    b = gu.run_gpu(inp, True)
    for n in ("dq_accum", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n


SPLIT = [(128, "bf16"), (128, "fp16"), (64, "bf16"), (16, "fp32"), (128, "fp32"), (32, "bf16")]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", SPLIT, ids=[f"{dt}-d{d}" for d, dt in SPLIT])
def test_split_passes_equal_fa_bwd(d, dtype, causal):
    """fa_bwd is exactly fa_bwd_dq followed by fa_bwd_dkdv, on every path."""
    import attention_fa_bwd_amd as fa
    gu.note(f"case split passes d={d} {dtype} causal={causal}")
    inp = si.draw_custom(1, 3, 700, d, dtype, seed=31)
    out = gu.run_gpu(inp, causal)
    q, k, v, do, L, D = (out[n] for n in ("q", "k", "v", "do", "L", "D"))
    dqa = torch.full_like(out["dq_accum"], float("nan"))
    dk, dv = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
    fa.fa_bwd_dq(q, k, v, do, L, D, dqa, inp.wl.scale, causal)
    fa.fa_bwd_dkdv(q, k, v, do, L, D, dk, dv, inp.wl.scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(dqa, out["dq_accum"])
    assert torch.equal(dk, out["dk"]) and torch.equal(dv, out["dv"])


@pytest.mark.parametrize("d,dtype", SPLIT, ids=[f"{dt}-d{d}" for d, dt in SPLIT])
def test_dq_accum_overwritten(d, dtype):
    """fa_bwd overwrites dq_accum: called twice on a buffer that holds the first
    call's result (or large values), it gives the same bits, never a sum."""
    import attention_fa_bwd_amd as fa
    gu.note(f"case dq_accum overwrite d={d} {dtype}")
    inp = si.draw_custom(2, 2, 260, d, dtype, seed=77)
    out = gu.run_gpu(inp, False)
    q, k, v, do, L, D = (out[n] for n in ("q", "k", "v", "do", "L", "D"))
    dqa, dk, dv = out["dq_accum"].clone(), torch.empty_like(q), torch.empty_like(q)
    fa.fa_bwd(q, k, v, do, L, D, dqa, dk, dv, inp.wl.scale, False)
    torch.cuda.synchronize()
    assert torch.equal(dqa, out["dq_accum"])
    dqa.fill_(1.0e6)
    fa.fa_bwd(q, k, v, do, L, D, dqa, dk, dv, inp.wl.scale, False)
    torch.cuda.synchronize()
    assert torch.equal(dqa, out["dq_accum"])


# ------------------------------------------------------ full-size workloads

# Whole heads compared element by element.  The heads cover different XCD
# shares of the work-item order and, under the causal mask, both heads of an
# interleaved pair: the bench shape's shares hold 4 heads each (pairs 0/1,
# 6/7, 18/19), the B=4 H=16 shares 8 each (pairs (0,0)/(0,1), (1,6)/(1,7),
# (2,8)/(2,9)); the long-context workload has 8 heads, one per share, all
# compared (in two halves, so that each test stays short).
WHOLE = {
    ("h32_n8192_d128_bf16", False): [[(0, 0), (0, 1), (0, 6), (0, 7), (0, 13), (0, 18), (0, 19), (0, 31)]],
    ("h32_n8192_d128_bf16", True): [[(0, 0), (0, 1), (0, 6), (0, 7), (0, 13), (0, 18), (0, 19), (0, 31)]],
    ("b4_h16_n4000_d128_bf16_q4", True): [[(0, 0), (0, 1), (0, 9), (1, 6), (1, 7), (2, 8), (2, 9), (3, 15)]],
    ("h8_n32768_d128_bf16", True): [[(0, 0), (0, 1), (0, 2), (0, 3)], [(0, 4), (0, 5), (0, 6), (0, 7)]],
}
WHOLE_CASES = [(n, c, i) for (n, c), parts in WHOLE.items() for i in range(len(parts))]
_full_cache = {}


@pytest.fixture(scope="module")
def full_runs():
    """GPU forward + backward of each full-size workload, computed once and
    shared by the tests of that workload; freed at the end of the module."""
    yield _full_cache
    _full_cache.clear()
    torch.cuda.empty_cache()


def _full_run(name, causal, dtype="bf16"):
    key = (name, causal, dtype)
    if key not in _full_cache:
        _full_cache.clear()
        torch.cuda.empty_cache()
        wl = si.WORKLOADS[name]
        gu.note(f"case {name} B={wl.B} H={wl.H} N={wl.N} d={wl.d} causal={causal} {dtype}: drawing")
        inp = si.draw(wl, dtype=dtype)
        gu.note("  running GPU forward + backward")
        out = gu.run_gpu(inp, causal)
        inv = gu.invariants(inp, causal, out)
        gu.note(f"  invariants over all heads {inv}")
        _full_cache[key] = (inp, out, inv)
    return _full_cache[key]


@pytest.mark.parametrize("name,causal,part", WHOLE_CASES,
                         ids=[f"{n}-{'causal' if c else 'full'}-{i}" for n, c, i in WHOLE_CASES])
def test_full_size_whole_heads(name, causal, part, full_runs):
    """Full problem sizes: every element of dQ, dK, dV of whole heads against
    the oracle's plain definition, and invariants over all heads."""
    inp, out, inv = _full_run(name, causal)
    assert not inv["nan"]
    assert inv["sum_dk"] <= 1e-2 and inv["sum_dv"] <= 1e-2
    if causal:
        assert inv["dq0"] <= 1e-3
    heads = WHOLE[(name, causal)][part]
    gu.note(f"  oracle on {len(heads)} whole heads")
    errs = gu.compare_heads(inp, causal, out, heads, log=gu.note)
    gu.note(f"  errs over the heads: dq {errs['dq']:.3e} dk {errs['dk']:.3e} dv {errs['dv']:.3e} "
            f"o {errs['o']:.3e} L {errs['L']:.3e}")
    _assert_grads(errs, gu.TOL["bf16"], name)
    assert errs["o"] <= gu.TOL["bf16"] and errs["L"] <= 1e-3


def test_full_size_fp16_sampled():
    """The bench shape in fp16 (the same contract): invariants over all heads,
    sampled rows of two heads against the oracle."""
    name, causal, dtype = "h32_n8192_d128_bf16", False, "fp16"
    wl = si.WORKLOADS[name]
    gu.note(f"case {name} causal={causal} {dtype}: drawing")
    inp = si.draw(wl, dtype=dtype)
    out = gu.run_gpu(inp, causal)
    inv = gu.invariants(inp, causal, out)
    gu.note(f"  invariants {inv}")
    assert not inv["nan"]
    assert inv["sum_dk"] <= 1e-2 and inv["sum_dv"] <= 1e-2
    errs = gu.compare_sampled(inp, causal, out, [(0, 0), (0, 31)])
    gu.note(f"  errs {errs}")
    _assert_grads(errs, gu.TOL[dtype], name)
    assert errs["o"] <= gu.TOL[dtype] and errs["L"] <= 1e-3
