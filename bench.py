#!/usr/bin/env python3
"""Benchmark of the FlashAttention-2 backward on one MI355X.

A step is one pass of the whole backward hot path -- fa_bwd_preprocess (D),
fa_bwd (the dQ and dK/dV passes; one launch on the matrix cores) and
fa_bwd_convert_dq -- over one batch of synthetic inputs already resident in
HBM.  The forward that
produces O and L runs once before timing and is not timed.

The line's value is the bench shape, B=1 H=32 N=8192 d=128 bf16 (non-causal
unless --causal).  Every other workload is timed with the same step and listed
under "configs", each with its own roofline entry and the oracle's CPU rate:
N=48 d=16 fp32 (both causal modes), B=1 H=8 N=1024 d=64 bf16, the bench
shape in both modes, B=4 H=16 N=4000 d=128 bf16 with Q x 4 (causal) and
B=1 H=8 N=32768 d=128 bf16 (causal).  FLOPs per step: 10*B*H*N^2*d, halved
under the causal mask.

Prints ONE JSON line.  Only one GPU is used; --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector: 256 CU x 2.4 GHz x 256 FLOP/clk
PEAK_HBM_GBS = 8000.0
METRIC = "attention backward TFLOP/s (10·B·H·N²·d, halved causal) and % bf16 MFMA peak"
MAIN_KERNEL_SOURCES = ["attention_fa_bwd_amd/csrc/bwd_dkdv.hpp", "attention_fa_bwd_amd/csrc/bwd_dq.hpp",
                       "attention_fa_bwd_amd/csrc/bwd_fused.hip", "attention_fa_bwd_amd/csrc/bwd_simt.hip",
                       "attention_fa_bwd_amd/csrc/mfma_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_bwd_main_traffic.json")
PRIMARY = "h32_n8192_d128_bf16"
# (workload, causal) of every timed configuration, in the order they run
CONFIGS = [("n48_d16_fp32", False), ("n48_d16_fp32", True), ("h8_n1024_d64_bf16", False),
           ("h32_n8192_d128_bf16", False), ("h32_n8192_d128_bf16", True),
           ("b4_h16_n4000_d128_bf16_q4", True), ("h8_n32768_d128_bf16", True)]
STEP_CALLS = ("fa_bwd_preprocess", "fa_bwd", "fa_bwd_convert_dq")


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=PRIMARY, choices=sorted({w for w, _ in CONFIGS}),
                   help="the workload of the line's value (the others are listed under configs)")
    p.add_argument("--causal", action="store_true", help="the line's value is the causal run")
    p.add_argument("--no-extra", action="store_true",
                   help="time only the line's own workload and mode (no other configs, no "
                        "forward / fa_lse / forward + backward lines)")
    p.add_argument("--no-other", action="store_true",
                   help="time only the line's own workload, in each of its causal modes")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="oracle time budget for the line's own workload (others: a third of it)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 512 MiB device copy (HBM counter calibration)")
    p.add_argument("--reference-gemm", action="store_true",
                   help="run only the library bf16 GEMM reference (for its counter profile)")
    return p.parse_args(argv)


def plan(args):
    """The (workload, causal) pairs one run times, the line's own first."""
    import seeded_inputs as si
    wl = si.WORKLOADS[args.workload]
    causal = bool(args.causal)
    if causal not in wl.causal:
        raise SystemExit(f"bench.py: workload {wl.name} runs causal={wl.causal}, not {causal}")
    first = (wl.name, causal)
    if args.no_extra:
        return [first]
    if args.no_other:
        return [first] + [(wl.name, c) for c in wl.causal if c != causal]
    return [first] + [c for c in CONFIGS if c != first]


def kernel_source_hash() -> str:
    """Hash of the backward kernels' code with comments and blank space removed,
    so that a comment edit does not invalidate counters taken on the same code."""
    h = hashlib.sha256()
    for rel in MAIN_KERNEL_SOURCES + ["attention_fa_bwd_amd/csrc/common.hpp"]:
        path = os.path.join(ROOT, rel)
        if os.path.exists(path):
            text = open(path, encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, causal: bool, kernel: str):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counter runs,
    or None when they are missing or were taken on other kernel sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    key = f"{kernel}/{workload}_{'causal' if causal else 'full'}"
    ent = rec.get("entries", {}).get(key)
    if not ent or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def calibrate_copy():
    import torch
    n = 512 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 5}))


# FLOPs per (b, h) as a multiple of N^2 d, before the causal halving.
# Algorithmic (the method's five products, FA2 chapter 16 sec 16.7: S, dP, dV,
# dK, dQ, 2 N^2 d each): fa_bwd does all five; of its two passes, the dK/dV
# pass forms S, dP, dV and dK (8) and the dQ pass forms dQ (2) -- its own S
# and dP are recomputation.  Executed (the products the kernels issue): the dQ
# pass forms S and dP again, 6 instead of 2, so fa_bwd issues 14.
KERNEL_FLOP_FACTOR = {"fa_bwd": 10.0, "fa_bwd_dkdv": 8.0, "fa_bwd_dq": 2.0}
EXECUTED_FLOP_FACTOR = {"fa_bwd": 14.0, "fa_bwd_dkdv": 8.0, "fa_bwd_dq": 6.0}


def elem_bytes(wl) -> int:
    return 4 if wl.dtype == "fp32" else 2


def hbm_kernel_bytes(wl) -> dict:
    """Algorithmic HBM bytes per launch of the two streaming steps."""
    rows, es = wl.B * wl.H * wl.N, elem_bytes(wl)
    return {"fa_bwd_preprocess": rows * wl.d * es * 2 + rows * 4,   # read O, dO; write D
            "fa_bwd_convert_dq": rows * wl.d * (4 + es)}            # read dq_accum; write dQ


def pass_flops(wl, causal: bool, kernel: str, executed: bool = False) -> float:
    factor = (EXECUTED_FLOP_FACTOR if executed else KERNEL_FLOP_FACTOR)[kernel]
    f = factor * wl.B * wl.H * wl.N * wl.N * wl.d
    return 0.5 * f if causal else f


def kernel_rates(wl, causal: bool, kernel: str, ms: float, peak: float) -> dict:
    """A kernel's rate on its algorithmic FLOPs (the roofline figures) and on
    the FLOPs it executes (how busy the unit is)."""
    kf, ke = pass_flops(wl, causal, kernel), pass_flops(wl, causal, kernel, executed=True)
    return {"avg_launch_ms": round(ms, 5), "flop_per_launch": kf,
            "achieved": round(kf / (ms * 1e-3) / 1e12, 3),
            "frac": round(kf / (ms * 1e-3) / 1e12 / peak, 4),
            "executed_flop_per_launch": ke,
            "executed_frac": round(ke / (ms * 1e-3) / 1e12 / peak, 4)}


def compute_peak(wl):
    """(bound, peak TFLOP/s) of the two passes: 16-bit inputs run on the
    matrix cores, fp32 on the vector ALUs (fp32 FMA)."""
    if wl.dtype == "fp32":
        return "alu", PEAK_FP32_VALU_TFLOPS
    return "mfma", PEAK_BF16_TFLOPS


def upload(inp):
    import numpy as np
    import torch
    if inp.wl.dtype == "fp32":
        return [torch.from_numpy(np.ascontiguousarray(getattr(inp, n))).cuda()
                for n in ("Q", "K", "V", "dO")]
    tdt = torch.bfloat16 if inp.wl.dtype == "bf16" else torch.float16
    return [torch.from_numpy(inp.bits[n].view(np.int16)).view(tdt).cuda()
            for n in ("Q", "K", "V", "dO")]


def gpu_time(wl, causal: bool, steps: int, warmup: int, inputs):
    import torch

    import attention_fa_bwd_amd as fa
    q, k, v, do, o, L = inputs
    B, H, N, d = q.shape
    scale = wl.scale
    D = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dqa = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()

    # one step: preprocess, fa_bwd (both passes), convert
    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.fa_bwd_preprocess(o, do, D, stream)
        if evs:
            evs[1].record(stream)
        fa.fa_bwd(q, k, v, do, L, D, dqa, dk, dv, scale, causal, stream)
        if evs:
            evs[2].record(stream)
        fa.fa_bwd_convert_dq(dqa, dq, scale, stream)
        if evs:
            evs[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K whole steps and nothing else on the stream, between two
    # HIP events (an event recorded between the calls costs a few microseconds,
    # which would weigh on the small workloads' steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    # the same K steps once more with HIP events on the launch stream between
    # the calls: each call's duration, and each step's
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    split = {name: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, name in enumerate(STEP_CALLS)}
    per_step = [e[0].elapsed_time(e[3]) for e in evs]
    return {
        "ms_per_step": total_ms / steps,
        "step_ms": {"median": round(statistics.median(per_step), 4),
                    "min": round(min(per_step), 4)},
        "wall_ms_per_step": 1e3 * wall / steps,
        "kernel_ms": {k: statistics.fmean(v) for k, v in split.items()},
        "kernel_ms_min": {k: min(v) for k, v in split.items()},
    }


def passes_alone(wl, causal: bool, inputs, reps: int = 5) -> dict:
    """Each pass launched on its own (fa_bwd_dq, fa_bwd_dkdv), outside the
    step: how fa_bwd's time splits between them."""
    import torch

    import attention_fa_bwd_amd as fa
    q, k, v, do, o, L = inputs
    B, H, N, d = q.shape
    D = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dqa = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()
    fa.fa_bwd_preprocess(o, do, D, stream)
    bound, peak = compute_peak(wl)
    out = {}
    for name, fn in (("fa_bwd_dq", lambda: fa.fa_bwd_dq(q, k, v, do, L, D, dqa, wl.scale, causal, stream)),
                     ("fa_bwd_dkdv", lambda: fa.fa_bwd_dkdv(q, k, v, do, L, D, dk, dv, wl.scale,
                                                            causal, stream))):
        out[name] = kernel_rates(wl, causal, name, timed_reps(fn, reps), peak)
    return out


def timed_reps(fn, reps: int = 5) -> float:
    """Mean ms of `reps` calls of fn on the current stream, after one warm-up."""
    import torch
    stream = torch.cuda.current_stream()
    fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def extras(wl, causal: bool, inputs, step_ms: float, flops: float) -> dict:
    """Beside the step, not part of it: the forward alone (with the backward /
    forward time ratio), L alone (fa_lse), and a whole training step of the
    attention (forward, then the backward step)."""
    import torch

    import attention_fa_bwd_amd as fa
    q, k, v, do = inputs
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    D = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dqa = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()
    s = wl.scale
    fms = timed_reps(lambda: fa.fa_fwd_lse(q, k, v, o, L, s, causal, stream))
    lms = timed_reps(lambda: fa.fa_lse(q, k, L, s, causal, stream))

    def train_step():
        fa.fa_fwd_lse(q, k, v, o, L, s, causal, stream)
        fa.fa_bwd_preprocess(o, do, D, stream)
        fa.fa_bwd(q, k, v, do, L, D, dqa, dk, dv, s, causal, stream)
        fa.fa_bwd_convert_dq(dqa, dq, s, stream)

    tms = timed_reps(train_step)
    ffl, lfl, tfl = 0.4 * flops, 0.2 * flops, 1.4 * flops  # 4, 2 and 14 N^2 d per head
    return {
        "forward": {"ms": round(fms, 4), "tflops": round(ffl / (fms * 1e-3) / 1e12, 3),
                    "bwd_over_fwd_time": round(step_ms / fms, 3)},
        "recompute_L": {"ms": round(lms, 4), "tflops": round(lfl / (lms * 1e-3) / 1e12, 3),
                        "step_ms_with_it": round(step_ms + lms, 4)},
        "forward_backward": {"ms": round(tms, 4), "tflops": round(tfl / (tms * 1e-3) / 1e12, 3)},
    }


def matmul_reference(n: int = 16384, reps: int = 5) -> dict:
    """A plain library bf16 GEMM (torch.matmul, dispatched to hipBLASLt) on the
    same GPU, timed like the kernels: the matrix-core rate a vendor-tuned dense
    product sustains on this device under load.  The backward's rate on the
    products it issues is read against it (a dense GEMM is the best case for
    the matrix cores: no softmax, no recomputation, no barriers per tile)."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    ms = timed_reps(lambda: torch.matmul(a, b, out=c), reps=reps)
    del a, b, c
    torch.cuda.empty_cache()
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"op": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt)", "ms": round(ms, 4),
            "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def cpu_host() -> str:
    model = "unknown CPU"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{len(os.sched_getaffinity(0))} CPUs usable of {os.cpu_count()}, {model}"


def cpu_baseline(wl, causal: bool, budget_s: float):
    """The oracle's full fp64 backward (by definition) on the host cores: whole
    heads of the workload, as many as fit in the time budget (at least one);
    problems whose every head takes well under the budget are repeated whole."""
    import numpy as np

    import oracle
    import seeded_inputs as si
    cores = oracle.max_threads()
    small = wl.B * wl.H * wl.N * wl.N * wl.d <= (1 << 31)
    sample = si.draw(wl) if small else si.draw(wl, B=1, H=1)
    Q, K, V, G = (np.ascontiguousarray(x, dtype=np.float64)
                  for x in (sample.Q, sample.K, sample.V, sample.dO))
    nheads = sample.Q.shape[0] * sample.Q.shape[1]
    heads, calls, elapsed = 0, 0, 0.0
    while elapsed < budget_s and (small or heads < wl.B * wl.H):
        t0 = time.perf_counter()
        oracle.attn_bwd(Q, K, V, G, wl.scale, causal)
        elapsed += time.perf_counter() - t0
        heads += nheads
        calls += 1
    flop = 10.0 * wl.N * wl.N * wl.d * (0.5 if causal else 1.0) * heads
    what = (f"the whole problem ({nheads} head(s)) {calls} time(s)" if small
            else f"{heads} of {wl.B * wl.H} head(s)")
    return {"value": flop / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} of N={wl.N}, d={wl.d} "
                      f"({'causal' if causal else 'non-causal'}), fp64 backward by definition, "
                      f"{elapsed:.2f} s",
            # the host the oracle ran on (hosts differ from one run to the next)
            "host": cpu_host()}


def bench_config(name: str, causal: bool, args, with_extras: bool, cpu_budget: float,
                 primary: bool):
    """Time the backward step on one workload and mode; per-kernel split,
    roofline of the dominant pass and (unless --no-cpu) the oracle's rate.
    The line's own workload is timed over exactly --steps steps; the other
    configurations whose step takes under a millisecond over at least 200, so
    that a single host-side delay between two launches of such a short step
    does not dominate the mean."""
    import torch

    import attention_fa_bwd_amd as fa
    import seeded_inputs as si
    wl = si.WORKLOADS[name]
    inp = si.draw(wl)
    q, k, v, do = upload(inp)
    del inp
    o, L = fa.forward(q, k, v, wl.scale, causal)
    torch.cuda.synchronize()
    steps, warmup = args.steps, args.warmup
    if not primary:
        # short steps: time at least ~100 ms after ~50 ms of warm-up, so that
        # the device has left its idle clocks (the oracle's CPU baseline of the
        # previous entry leaves it idle for seconds) and one host-side delay
        # does not dominate the mean
        probe = gpu_time(wl, causal, 3, 1, (q, k, v, do, o, L))
        per = probe["step_ms"]["median"]
        if per < 1.0:
            steps = max(steps, 200, int(100.0 / per))
            warmup = max(warmup, int(50.0 / per))
    r = gpu_time(wl, causal, steps, warmup, (q, k, v, do, o, L))
    flops = wl.flops(causal)
    tflops = flops / (r["ms_per_step"] * 1e-3) / 1e12
    bound, peak = compute_peak(wl)
    kernels = {}
    kernels["fa_bwd"] = kernel_rates(wl, causal, "fa_bwd", r["kernel_ms"]["fa_bwd"], peak)
    for kname, nbytes in hbm_kernel_bytes(wl).items():
        ms = r["kernel_ms"][kname]
        gbs = nbytes / (ms * 1e-3) / 1e9
        kernels[kname] = {"avg_launch_ms": round(ms, 5), "bytes_per_launch": nbytes,
                          "achieved_gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    dom = "fa_bwd"   # the main step: far longer than preprocess and convert
    kd = kernels[dom]
    alone = passes_alone(wl, causal, (q, k, v, do, o, L))
    out = {
        "workload": f"B={wl.B} H={wl.H} N={wl.N} d={wl.d} {wl.dtype}"
                    f"{' Q x %g' % wl.q_mult if wl.q_mult != 1.0 else ''} "
                    f"{'causal' if causal else 'non-causal'}",
        "name": wl.name, "causal": causal, "dtype": wl.dtype,
        "flop_per_step": flops, "steps": steps, "warmup": warmup,
        "value": round(tflops, 4), "unit": "TFLOP/s",
        "ms_per_step": round(r["ms_per_step"], 5),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 3),
        "step_ms": r["step_ms"],
        "split_ms": {kk: round(vv, 5) for kk, vv in r["kernel_ms"].items()},
        "split_method": "a second pass of the same steps with HIP events between the calls",
        "roofline": {"bound": bound, "kernel": dom, "achieved": kd["achieved"], "peak": peak,
                     "unit": "TFLOP/s", "frac": kd["frac"],
                     "traffic": load_traffic(wl.name, causal, dom),
                     "flop_per_launch": kd["flop_per_launch"],
                     "avg_launch_ms": kd["avg_launch_ms"],
                     "executed_frac": kd["executed_frac"]},
        "kernels": kernels,
        "passes_alone": alone,
    }
    if with_extras:
        out.update(extras(wl, causal, (q, k, v, do), r["ms_per_step"], flops))
    del q, k, v, do, o, L
    torch.cuda.empty_cache()
    out["cpu_baseline"] = None if args.no_cpu else cpu_baseline(wl, causal, cpu_budget)
    print(f"bench.py: {out['workload']}: {out['value']:.1f} TFLOP/s, "
          f"{out['ms_per_step']:.4f} ms per step", file=sys.stderr, flush=True)
    return out


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "heads shard across GPUs with no communication, see the design notes.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.reference_gemm:
        print(json.dumps({"matmul_reference": matmul_reference()}), flush=True)
        return
    runs = plan(args)
    results = []
    for i, (name, causal) in enumerate(runs):
        results.append(bench_config(name, causal, args,
                                    with_extras=(name == PRIMARY and not args.no_extra),
                                    cpu_budget=args.cpu_seconds if i == 0 else args.cpu_seconds / 3,
                                    primary=(i == 0)))
    prim = results[0]
    import seeded_inputs as si
    wl = si.WORKLOADS[prim["name"]]
    line = {
        "metric": METRIC,
        "value": round(prim["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prim["dtype"],
        "data": "synthetic (seeded standard normal Q, K, V, dO)",
        "config": {"workload": prim["workload"], "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "causal": prim["causal"], "parallelism": "single GPU"},
        "pct_bf16_peak": round(prim["pct_bf16_peak"], 2),
        "step_ms": prim["step_ms"],
        "split_ms": prim["split_ms"],
        "roofline": prim["roofline"],
        "kernels": prim["kernels"],
    }
    for key in ("forward", "recompute_L", "forward_backward"):
        if key in prim:
            line[key] = prim[key]
    if not args.no_extra:
        ref = matmul_reference()
        fb = prim["kernels"]["fa_bwd"]
        # the backward's products issued per second over the library GEMM's
        ref["fa_bwd_executed_over_matmul"] = round(
            fb["executed_flop_per_launch"] / (fb["avg_launch_ms"] * 1e-3) / 1e12 / ref["tflops"], 3)
        line["matmul_reference"] = ref
    line["cpu_baseline"] = prim["cpu_baseline"]
    line["configs"] = results
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
