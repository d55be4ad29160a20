"""fa_bwd_noalloc on the GPU, through the C ABI: its dQ, dK and dV against the
existing entry points (fa_bwd_preprocess, fa_bwd, fa_bwd_convert_dq) on the
same inputs -- bit for bit, which is stricter than the oracle bar -- and
against the oracle within the bar.  Two calls in a row per case, the second
on a smaller problem, so the second call reuses the scratch array the first
one filled."""
import pytest
import torch

import seeded_inputs as si

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_util as gu
    import attention_fa_bwd_amd as fa
else:  # collected on CPU-only machines, never run there
    gu = fa = None

CASES = [(128, "bf16"), (128, "fp16"), (64, "bf16"), (64, "fp16"), (16, "fp32"), (32, "bf16")]
SIZES = [(2, 3, 700), (1, 2, 130)]   # first call, then a smaller second call


def _noalloc(out, inp, causal):
    dq, dk, dv = (torch.full_like(out["q"], float("nan")) for _ in range(3))
    fa.fa_bwd_noalloc(out["q"], out["k"], out["v"], out["o"], out["do"], out["L"], dq, dk, dv,
                      inp.wl.scale, causal)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", CASES, ids=[f"{dt}-d{d}" for d, dt in CASES])
def test_noalloc_equals_three_calls(d, dtype, causal):
    for i, (B, H, N) in enumerate(SIZES):
        gu.note(f"case noalloc {dtype} d={d} causal={causal} call {i + 1}: B={B} H={H} N={N}")
        inp = si.draw_custom(B, H, N, d, dtype, seed=1300 + 10 * i + d)
        out = gu.run_gpu(inp, causal)          # forward, then the three existing calls
        dq, dk, dv = _noalloc(out, inp, causal)
        assert torch.equal(dq, out["dq"]), "dQ differs from fa_bwd + fa_bwd_convert_dq"
        assert torch.equal(dk, out["dk"]) and torch.equal(dv, out["dv"])
        errs = gu.compare_full(inp, causal, dict(out, dq=dq, dk=dk, dv=dv))
        for n in ("dq", "dk", "dv"):
            assert errs[n] <= gu.TOL[dtype], f"{n} rel err {errs[n]:.3e}"


def test_noalloc_full_size_bench_shape():
    """The bench shape (B=1 H=32 N=8192 d=128 bf16, 262144 rows of D in the
    scratch array), then a small problem after it."""
    for causal, (B, H, N, d) in ((False, (1, 32, 8192, 128)), (True, (1, 3, 517, 128))):
        gu.note(f"case noalloc full size B={B} H={H} N={N} causal={causal}")
        inp = si.draw_custom(B, H, N, d, "bf16", seed=1400 + N)
        out = gu.run_gpu(inp, causal)
        dq, dk, dv = _noalloc(out, inp, causal)
        assert torch.equal(dq, out["dq"])
        assert torch.equal(dk, out["dk"]) and torch.equal(dv, out["dv"])
