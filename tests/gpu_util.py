"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI binding, and compare with the fp64 oracle.

Error measure (per gradient tensor): max |g_gpu - g_ref| / max |g_ref| over the
compared elements -- the whole tensor where the oracle computes it whole, the
sampled rows of the sampled heads at full problem sizes.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import attention_fa_bwd_amd as fa
import oracle
import seeded_inputs as si

TOL = {"fp32": 1e-5, "bf16": 2e-2, "fp16": 1e-2}
TORCH_DT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def note(msg: str) -> None:
    """Print and flush a line naming the case before GPU work starts."""
    print(msg, flush=True)
    sys.stdout.flush()


def upload(inp: si.Inputs, name: str) -> torch.Tensor:
    if inp.wl.dtype in ("bf16", "fp16"):
        b = np.ascontiguousarray(inp.bits[name]).view(np.int16)
        return torch.from_numpy(b).view(TORCH_DT[inp.wl.dtype]).cuda()
    return torch.from_numpy(np.ascontiguousarray(getattr(inp, name))).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.abs(ref).max())
    num = float(np.abs(gpu - ref).max())
    return num / den if den > 0 else num


def run_gpu(inp: si.Inputs, causal: bool, O=None, L=None):
    """Forward (unless O, L are given) then the three backward calls.

    Returns dict of device tensors: o, L, dq, dk, dv, D, dq_accum."""
    q, k, v, do = (upload(inp, n) for n in ("Q", "K", "V", "dO"))
    scale = inp.wl.scale
    if O is None:
        o, Lt = fa.forward(q, k, v, scale, causal)
    else:
        o = torch.from_numpy(np.ascontiguousarray(O)).to(TORCH_DT[inp.wl.dtype]).cuda()
        Lt = torch.from_numpy(np.ascontiguousarray(L, dtype=np.float32)).cuda()
    B, H, N, d = q.shape
    D = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    dqa = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.fa_bwd_preprocess(o, do, D)
    fa.fa_bwd(q, k, v, do, Lt, D, dqa, dk, dv, scale, causal)
    fa.fa_bwd_convert_dq(dqa, dq, scale)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, do=do, o=o, L=Lt, dq=dq, dk=dk, dv=dv, D=D, dq_accum=dqa)


def compare_full(inp: si.Inputs, causal: bool, out: dict) -> dict:
    """Whole-tensor comparison with the oracle's definitions."""
    scale = inp.wl.scale
    dQ, dK, dV, D = oracle.attn_bwd(inp.Q, inp.K, inp.V, inp.dO, scale, causal)
    O, L = oracle.attn_fwd(inp.Q, inp.K, inp.V, scale, causal)
    errs = {
        "dq": rel_err(to_f64(out["dq"]), dQ),
        "dk": rel_err(to_f64(out["dk"]), dK),
        "dv": rel_err(to_f64(out["dv"]), dV),
        "o": rel_err(to_f64(out["o"]), O),
        "L": float(np.abs(to_f64(out["L"]) - L).max()),
        "D": rel_err(to_f64(out["D"]), D),
    }
    return errs


def sample_rows(N: int, n: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, N // 2, N - 2, N - 1]
    extra = rng.choice(N, size=min(n, N), replace=False).tolist()
    return sorted(set(r for r in fixed + extra if 0 <= r < N))


def compare_sampled(inp: si.Inputs, causal: bool, out: dict, heads, nrows: int = 24) -> dict:
    """Compare sampled rows of sampled (b, h) heads with the oracle.

    For each head the oracle computes every row's L and D by definition, then dQ
    of the sampled rows and dK, dV of the sampled keys, plus O and L of the
    sampled rows for the forward."""
    scale = inp.wl.scale
    N = inp.wl.N
    acc = {n: [[], []] for n in ("dq", "dk", "dv", "o")}
    lerr = 0.0
    for (b, h) in heads:
        Q, K, V, G = (np.ascontiguousarray(getattr(inp, n)[b, h], dtype=np.float64)
                      for n in ("Q", "K", "V", "dO"))
        rows = sample_rows(N, nrows, seed=1000 * b + h)
        Lr, Dr = oracle.row_stats(Q, K, V, G, scale, causal)
        dq = oracle.dq_rows(Q, K, V, G, scale, causal, rows)
        dk, dv = oracle.dkdv_rows(Q, K, V, G, Lr, Dr, scale, causal, rows)
        o, l = oracle.fwd_rows(Q, K, V, scale, causal, rows)
        idx = torch.tensor(rows, device="cuda")
        for name, ref in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o)):
            acc[name][0].append(to_f64(out[name][b, h].index_select(0, idx)))
            acc[name][1].append(ref)
        lerr = max(lerr, float(np.abs(to_f64(out["L"][b, h].index_select(0, idx)) - l).max()))
    errs = {n: rel_err(np.concatenate(a[0]), np.concatenate(a[1])) for n, a in acc.items()}
    errs["L"] = lerr
    return errs


def compare_heads(inp: si.Inputs, causal: bool, out: dict, heads, log=None) -> dict:
    """Every element of dQ, dK, dV and O of whole (b, h) heads against the
    oracle's plain definitions (oracle.attn_bwd and attn_fwd on that head
    alone), and L as the largest absolute difference.  Returns the error
    measure over all compared elements per tensor, and per head."""
    scale = inp.wl.scale
    acc = {n: [0.0, 0.0] for n in ("dq", "dk", "dv", "o")}   # max |err|, max |ref|
    per_head = {}
    lerr = 0.0
    for (b, h) in heads:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, h:h + 1], dtype=np.float64)
        dQ, dK, dV, _ = oracle.attn_bwd(sl(inp.Q), sl(inp.K), sl(inp.V), sl(inp.dO), scale, causal)
        O, L = oracle.attn_fwd(sl(inp.Q), sl(inp.K), sl(inp.V), scale, causal)
        lerr = max(lerr, float(np.abs(to_f64(out["L"][b:b + 1, h:h + 1]) - L).max()))
        errs = {}
        for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV), ("o", O)):
            g = to_f64(out[name][b:b + 1, h:h + 1])
            num, den = float(np.abs(g - ref).max()), float(np.abs(ref).max())
            acc[name][0] = max(acc[name][0], num)
            acc[name][1] = max(acc[name][1], den)
            errs[name] = num / den if den > 0 else num
        per_head[(b, h)] = errs
        if log:
            log(f"  head ({b},{h}): " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    res = {n: (a[0] / a[1] if a[1] > 0 else a[0]) for n, a in acc.items()}
    res["L"] = lerr
    res["per_head"] = per_head
    return res


def invariants(inp: si.Inputs, causal: bool, out: dict) -> dict:
    """Properties exact in real arithmetic, checked on whole GPU outputs:
    sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, and (causal) dQ_0 = 0."""
    dk = out["dk"].double()
    dv = out["dv"].double()
    do = out["do"].double()
    dq = out["dq"].double()
    r = {
        "sum_dk": float(dk.sum(2).abs().max() / dk.abs().sum(2).max()),
        "sum_dv": float((dv.sum(2) - do.sum(2)).abs().max() / dv.abs().sum(2).max()),
    }
    if causal:
        r["dq0"] = float(dq[:, :, 0].abs().max() / dq.abs().max())
    r["nan"] = bool(torch.isnan(dq).any() or torch.isnan(dk).any() or torch.isnan(dv).any())
    return r


def flops_note(inp: si.Inputs, causal: bool) -> float:
    return inp.wl.flops(causal) / 1e12


__all__ = ["TOL", "note", "upload", "to_f64", "rel_err", "run_gpu", "compare_full",
           "compare_sampled", "compare_heads", "invariants", "sample_rows", "flops_note", "math"]
