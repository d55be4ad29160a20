"""The stream and shape contract of the C ABI on the GPU.

* Calls only enqueue on the stream they are given, and calls on different
  streams with disjoint buffers may run concurrently: two independent
  backward problems issued alternately on two streams give the same results
  as the same calls issued one problem after the other, bitwise (no path
  uses atomics).
* Many heads: thousands of (b, h) pairs of a short sequence exercise the
  work-item decomposition of every kernel; sampled heads are compared with
  the oracle's plain definition."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import seeded_inputs as si
import attention_fa_bwd_amd as fa

pytestmark = pytest.mark.gpu


def _problem(inp, causal, stream):
    """Device tensors plus the full forward + backward enqueued on `stream`."""
    with torch.cuda.stream(stream):
        q, k, v, do = (gu.upload(inp, n) for n in ("Q", "K", "V", "dO"))
    stream.synchronize()
    B, H, N, d = q.shape
    t = dict(q=q, k=k, v=v, do=do,
             o=torch.empty_like(q), L=torch.empty((B, H, N), dtype=torch.float32, device="cuda"),
             D=torch.empty((B, H, N), dtype=torch.float32, device="cuda"),
             dqa=torch.empty((B, H, N, d), dtype=torch.float32, device="cuda"),
             dq=torch.empty_like(q), dk=torch.empty_like(q), dv=torch.empty_like(q))
    scale = inp.wl.scale
    calls = [
        lambda: fa.fa_fwd_lse(t["q"], t["k"], t["v"], t["o"], t["L"], scale, causal, stream),
        lambda: fa.fa_bwd_preprocess(t["o"], t["do"], t["D"], stream),
        lambda: fa.fa_bwd(t["q"], t["k"], t["v"], t["do"], t["L"], t["D"], t["dqa"], t["dk"],
                          t["dv"], scale, causal, stream),
        lambda: fa.fa_bwd_convert_dq(t["dqa"], t["dq"], scale, stream),
    ]
    return t, calls


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 128), ("bf16", 64), ("fp32", 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_two_streams_match_one(dtype, d, causal):
    gu.note(f"case two streams {dtype} d={d} causal={causal}")
    ia = si.draw_custom(2, 3, 777, d, dtype, seed=901)
    ib = si.draw_custom(1, 5, 513, d, dtype, seed=902)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    # reference: each problem alone, one after the other on one stream
    ref = []
    for inp in (ia, ib):
        t, calls = _problem(inp, causal, s1)
        for c in calls:
            c()
        s1.synchronize()
        ref.append({n: t[n].clone() for n in ("o", "L", "dq", "dk", "dv")})
    # the same calls interleaved across two streams
    ta, ca = _problem(ia, causal, s1)
    tb, cb = _problem(ib, causal, s2)
    for x, y in zip(ca, cb):
        x()
        y()
    s1.synchronize()
    s2.synchronize()
    for t, r in ((ta, ref[0]), (tb, ref[1])):
        for n in ("o", "L", "dq", "dk", "dv"):
            assert torch.equal(t[n], r[n]), n


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_many_heads(dtype):
    """B x H = 3 x 1100 heads of N = 70 (d = 128): 3300 work items per pass,
    a ragged last tile in every one."""
    gu.note(f"case many heads {dtype}")
    inp = si.draw_custom(3, 1100, 70, 128, dtype, seed=903)
    causal = True
    out = gu.run_gpu(inp, causal)
    rng = np.random.default_rng(5)
    heads = [(0, 0), (2, 1099)] + [(int(b), int(h)) for b, h in
                                   zip(rng.integers(0, 3, 4), rng.integers(0, 1100, 4))]
    for b, h in heads:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, h:h + 1])
        dQ, dK, dV, _ = oracle.attn_bwd(sl(inp.Q), sl(inp.K), sl(inp.V), sl(inp.dO),
                                        inp.wl.scale, causal)
        for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
            err = gu.rel_err(gu.to_f64(out[name][b:b + 1, h:h + 1]), ref)
            assert err <= gu.TOL[dtype], f"head ({b},{h}) {name} {err:.3e}"
