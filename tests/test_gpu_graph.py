"""HIP graph capture of the C ABI on the GPU.

The library allocates nothing, clears no memory with a memset and never
synchronises inside a call, so a caller can capture a whole attention training
step -- forward, preprocess, both backward passes, convert -- or the
no-allocation backward into a HIP graph and replay it.  Each test warms the
calls up eagerly (the library's one-time device queries), captures them on a
side stream, and replays the graph several times with the program's own eager
work between replays (outputs poisoned with NaN, inputs rewritten) and a
synchronisation after each; every replay is compared bitwise with the same
calls run eagerly on the same inputs."""
import pytest
import torch

import gpu_util as gu
import seeded_inputs as si
import attention_fa_bwd_amd as fa

pytestmark = pytest.mark.gpu

CASES = [(128, "bf16", False), (128, "bf16", True), (64, "fp16", True), (16, "fp32", False)]


def _tensors(inp):
    q, k, v, do = (gu.upload(inp, n) for n in ("Q", "K", "V", "dO"))
    B, H, N, d = q.shape
    f32 = dict(dtype=torch.float32, device="cuda")
    return dict(q=q, k=k, v=v, do=do, o=torch.empty_like(q), L=torch.empty((B, H, N), **f32),
                D=torch.empty((B, H, N), **f32), dqa=torch.empty((B, H, N, d), **f32),
                dq=torch.empty_like(q), dk=torch.empty_like(q), dv=torch.empty_like(q))


def _capture(fn):
    """fn(stream) captured into a graph on a side stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        fn(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _replays(g, eager, t, outs, rewrite):
    """Replays of g against eager runs: the same inputs, then rewritten ones."""
    for rep in range(4):
        if rep == 2:
            rewrite()
        eager(torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref = {n: t[n].clone() for n in outs}
        for n in outs:
            t[n].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(t[n], ref[n]), f"replay {rep}: {n} differs from the eager call"


@pytest.mark.parametrize("d,dtype,causal", CASES, ids=[f"{dt}-d{d}-c{int(c)}" for d, dt, c in CASES])
def test_training_step_graph_replays(d, dtype, causal):
    gu.note(f"case graph training step {dtype} d={d} causal={causal}")
    inp = si.draw_custom(1, 4, 700, d, dtype, seed=2100 + d)
    t = _tensors(inp)
    scale = inp.wl.scale

    def step(stream):
        fa.fa_fwd_lse(t["q"], t["k"], t["v"], t["o"], t["L"], scale, causal, stream)
        fa.fa_bwd_preprocess(t["o"], t["do"], t["D"], stream)
        fa.fa_bwd(t["q"], t["k"], t["v"], t["do"], t["L"], t["D"], t["dqa"], t["dk"], t["dv"],
                  scale, causal, stream)
        fa.fa_bwd_convert_dq(t["dqa"], t["dq"], scale, stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = _capture(step)
    _replays(g, step, t, ("o", "L", "D", "dqa", "dq", "dk", "dv"),
             lambda: (t["q"].mul_(0.5), t["do"].neg_()))


@pytest.mark.parametrize("d,dtype,causal", CASES, ids=[f"{dt}-d{d}-c{int(c)}" for d, dt, c in CASES])
def test_noalloc_backward_graph_replays(d, dtype, causal):
    gu.note(f"case graph no-allocation backward {dtype} d={d} causal={causal}")
    inp = si.draw_custom(1, 4, 700, d, dtype, seed=2200 + d)
    t = _tensors(inp)
    scale = inp.wl.scale
    fa.fa_fwd_lse(t["q"], t["k"], t["v"], t["o"], t["L"], scale, causal)
    torch.cuda.synchronize()

    def bwd(stream):
        fa.fa_bwd_noalloc(t["q"], t["k"], t["v"], t["o"], t["do"], t["L"], t["dq"], t["dk"],
                          t["dv"], scale, causal, stream)

    bwd(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = _capture(bwd)
    _replays(g, bwd, t, ("dq", "dk", "dv"), lambda: t["do"].mul_(2.0))
