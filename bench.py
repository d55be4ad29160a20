#!/usr/bin/env python3
"""Benchmark of the FlashAttention-2 backward on one MI355X.

A step is one pass of the whole backward hot path -- fa_bwd_preprocess (D),
the two passes of fa_bwd (fa_bwd_dq, then fa_bwd_dkdv) and fa_bwd_convert_dq --
over one batch of synthetic inputs already resident in HBM.  The forward that produces O and
L runs once before timing and is not timed.

Workload (default): B=1, H=32, N=8192, d=128, bf16, non-causal; the causal
variant of the same shape is timed too and reported under "causal", and the
same step is timed on the two other full-size workloads (B=4 H=16 N=4000 with
Q scaled by 4, and B=1 H=8 N=32768, both causal) under "other_workloads".
FLOPs per step: 10*B*H*N^2*d, halved under the causal mask.

Prints ONE JSON line.  Only one GPU is used; --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
METRIC = "attention backward TFLOP/s (10·B·H·N²·d, halved causal) and % bf16 MFMA peak"
MAIN_KERNEL_SOURCES = ["attention_fa_bwd_amd/csrc/bwd_dkdv.hip", "attention_fa_bwd_amd/csrc/bwd_dq.hip", "attention_fa_bwd_amd/csrc/mfma_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_bwd_main_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="h32_n8192_d128_bf16",
                   choices=["h8_n1024_d64_bf16", "h32_n8192_d128_bf16",
                            "b4_h16_n4000_d128_bf16_q4", "h8_n32768_d128_bf16"])
    p.add_argument("--causal", action="store_true", help="primary line is the causal run")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the second causal mode and the other workloads")
    p.add_argument("--no-other", action="store_true",
                   help="skip the other workloads (both causal modes of the main one still run)")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 512 MiB device copy (HBM counter calibration)")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the main kernels' code with comments and blank space removed, so
    that a comment edit does not invalidate counters taken on the same code."""
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


# Algorithmic FLOPs of each backward kernel per (b, h), before the causal halving:
# the dK/dV pass recomputes S and dP and forms dV and dK (4 of the 5 products),
# the dQ pass recomputes S and dP and forms dQ (3 products).
KERNEL_FLOP_FACTOR = {"fa_bwd_dkdv": 8.0, "fa_bwd_dq": 6.0}


def hbm_kernel_bytes(wl) -> dict:
    """Algorithmic HBM bytes per launch of the two streaming steps (16-bit
    elements, d = 128: the preprocess leaves dq_accum to the dQ pass)."""
    rows = wl.B * wl.H * wl.N
    return {"fa_bwd_preprocess": rows * wl.d * 2 * 2 + rows * 4,   # read O, dO; write D
            "fa_bwd_convert_dq": rows * wl.d * (4 + 2)}           # read dq_accum; write dQ


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

    # one step: preprocess, dQ pass, dK/dV pass, convert (fa_bwd runs the two
    # passes back to back; calling them separately lets events split them)
    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.fa_bwd_preprocess(o, do, D, stream)
        if evs:
            evs[1].record(stream)
        fa.fa_bwd_dq(q, k, v, do, L, D, dqa, scale, causal, stream)
        if evs:
            evs[2].record(stream)
        fa.fa_bwd_dkdv(q, k, v, do, L, D, dk, dv, scale, causal, stream)
        if evs:
            evs[3].record(stream)
        fa.fa_bwd_convert_dq(dqa, dq, scale, stream)
        if evs:
            evs[4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K whole steps; HIP events on the launch stream split it per kernel
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    split = {name: [e[j].elapsed_time(e[j + 1]) for e in evs]
             for j, name in enumerate(("fa_bwd_preprocess", "fa_bwd_dq", "fa_bwd_dkdv",
                                       "fa_bwd_convert_dq"))}
    per_step = [e[0].elapsed_time(e[4]) for e in evs]
    return {
        "ms_per_step": total_ms / steps,
        "step_ms": {"median": round(statistics.median(per_step), 4),
                    "min": round(min(per_step), 4)},
        "wall_ms_per_step": 1e3 * wall / steps,
        "kernel_ms": {k: statistics.fmean(v) for k, v in split.items()},
        "kernel_ms_min": {k: min(v) for k, v in split.items()},
    }


def forward_time(wl, causal: bool, inputs, reps: int = 5):
    """Time of the forward alone (not part of a step): HIP events around
    `reps` calls on the launch stream after one warm-up call."""
    import torch

    import attention_fa_bwd_amd as fa
    q, k, v = inputs
    o = torch.empty_like(q)
    L = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fa.fa_fwd_lse(q, k, v, o, L, wl.scale, causal, stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fa.fa_fwd_lse(q, k, v, o, L, wl.scale, causal, stream)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def lse_time(wl, causal: bool, inputs, reps: int = 5):
    """Time of fa_lse alone (L recomputed when the forward did not keep it;
    not part of a step): HIP events around `reps` calls after one warm-up."""
    import torch

    import attention_fa_bwd_amd as fa
    q, k = inputs
    L = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fa.fa_lse(q, k, L, wl.scale, causal, stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fa.fa_lse(q, k, L, wl.scale, causal, stream)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def fwd_bwd_time(wl, causal: bool, inputs, reps: int = 5):
    """Time of a whole training step of the attention (not the metric's
    step): fa_fwd_lse, then the backward (preprocess, both passes, convert),
    all on the launch stream; HIP events around `reps` steps after a warm-up."""
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

    def one():
        fa.fa_fwd_lse(q, k, v, o, L, wl.scale, causal, stream)
        fa.fa_bwd_preprocess(o, do, D, stream)
        fa.fa_bwd(q, k, v, do, L, D, dqa, dk, dv, wl.scale, causal, stream)
        fa.fa_bwd_convert_dq(dqa, dq, wl.scale, stream)

    one()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        one()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def cpu_baseline(wl, causal: bool, budget_s: float):
    """The oracle's full backward (by definition) on a bounded sample of heads."""
    import numpy as np

    import oracle
    import seeded_inputs as si
    cores = oracle.max_threads()
    sample = si.draw(wl, B=1, H=1)             # same shape per head, same recipe
    Q, K, V, G = (np.ascontiguousarray(x, dtype=np.float64) for x in (sample.Q, sample.K, sample.V, sample.dO))
    heads, elapsed = 0, 0.0
    while elapsed < budget_s and heads < wl.B * wl.H:
        t0 = time.perf_counter()
        oracle.attn_bwd(Q, K, V, G, wl.scale, causal)
        elapsed += time.perf_counter() - t0
        heads += 1
    flop = 10.0 * wl.N * wl.N * wl.d * (0.5 if causal else 1.0) * heads
    model = "unknown CPU"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flop / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} head(s) of N={wl.N}, d={wl.d} ({'causal' if causal else 'non-causal'}), "
                      f"fp64 backward by definition, {elapsed:.1f} s",
            # the host the oracle ran on (hosts differ from one run to the next)
            "host": f"{len(os.sched_getaffinity(0))} CPUs usable of {os.cpu_count()}, {model}"}


def other_workload(wl, args):
    """One backward step timed on another workload, in each of its causal modes."""
    import numpy as np
    import torch

    import attention_fa_bwd_amd as fa
    import seeded_inputs as si
    inp = si.draw(wl)
    up = [torch.from_numpy(inp.bits[n].view(np.int16)).view(torch.bfloat16).cuda()
          for n in ("Q", "K", "V", "dO")]
    out = {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "modes": []}
    for causal in wl.causal:
        o, L = fa.forward(up[0], up[1], up[2], wl.scale, causal)
        torch.cuda.synchronize()
        r = gpu_time(wl, causal, args.steps, args.warmup, (*up, o, L))
        tf = wl.flops(causal) / (r["ms_per_step"] * 1e-3) / 1e12
        out["modes"].append({"causal": causal, "ms_per_step": round(r["ms_per_step"], 4),
                             "tflops": round(tf, 3),
                             "pct_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
                             "split_ms": {k: round(v, 4) for k, v in r["kernel_ms"].items()}})
        del o, L
    del up
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "heads shard across GPUs with no communication, see the design notes.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import attention_fa_bwd_amd as fa
    import seeded_inputs as si

    if args.calibrate_copy:
        calibrate_copy()
        return
    wl = si.WORKLOADS[args.workload]
    modes = [args.causal] if args.no_extra else [args.causal, not args.causal]
    modes = [m for m in modes if m in (False, True)]
    inp = si.draw(wl)
    up = {n: torch.from_numpy(inp.bits[n].view(np.int16)).view(torch.bfloat16).cuda()
          for n in ("Q", "K", "V", "dO")}
    results = {}
    for causal in modes:
        o, L = fa.forward(up["Q"], up["K"], up["V"], wl.scale, causal)
        torch.cuda.synchronize()
        r = gpu_time(wl, causal, args.steps, args.warmup, (up["Q"], up["K"], up["V"], up["dO"], o, L))
        flops = wl.flops(causal)
        r["tflops"] = flops / (r["ms_per_step"] * 1e-3) / 1e12
        r["pct_peak"] = 100.0 * r["tflops"] / PEAK_BF16_TFLOPS
        r["kernels"] = {}
        for name, fac in KERNEL_FLOP_FACTOR.items():
            kflop = fac / 10.0 * flops
            ms = r["kernel_ms"][name]
            r["kernels"][name] = {"avg_launch_ms": round(ms, 4), "flop_per_launch": kflop,
                                  "achieved": round(kflop / (ms * 1e-3) / 1e12, 3),
                                  "frac": round(kflop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        for name, nbytes in hbm_kernel_bytes(wl).items():
            ms = r["kernel_ms"][name]
            gbs = nbytes / (ms * 1e-3) / 1e9
            r["kernels"][name] = {"avg_launch_ms": round(ms, 4), "bytes_per_launch": nbytes,
                                  "achieved_gbs": round(gbs, 1),
                                  "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        fms = forward_time(wl, causal, (up["Q"], up["K"], up["V"]))
        ffl = 0.4 * flops  # 4·B·H·N²·d (×½ causal)
        r["forward"] = {"ms": round(fms, 4), "tflops": round(ffl / (fms * 1e-3) / 1e12, 3),
                        "bwd_over_fwd_time": round(r["ms_per_step"] / fms, 3)}
        lms = lse_time(wl, causal, (up["Q"], up["K"]))
        lfl = 0.2 * flops  # S only: 2·B·H·N²·d (×½ causal)
        r["recompute_L"] = {"ms": round(lms, 4), "tflops": round(lfl / (lms * 1e-3) / 1e12, 3),
                            "step_ms_with_it": round(r["ms_per_step"] + lms, 4)}
        tms = fwd_bwd_time(wl, causal, (up["Q"], up["K"], up["V"], up["dO"]))
        tfl = 1.4 * flops  # forward 4 + backward 10: 14·B·H·N²·d (×½ causal)
        r["forward_backward"] = {"ms": round(tms, 4),
                                 "tflops": round(tfl / (tms * 1e-3) / 1e12, 3)}
        results[causal] = r
        del o, L
    prim = results[args.causal]
    dom = max(KERNEL_FLOP_FACTOR, key=lambda n: prim["kernel_ms"][n])
    kd = prim["kernels"][dom]
    line = {
        "metric": METRIC,
        "value": round(prim["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded standard normal Q, K, V, dO)",
        "config": {"workload": f"B={wl.B} H={wl.H} N={wl.N} d={wl.d} bf16 "
                               f"{'causal' if args.causal else 'non-causal'}",
                   "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "causal": args.causal,
                   "parallelism": "single GPU"},
        "pct_bf16_peak": round(prim["pct_peak"], 2),
        "step_ms": prim["step_ms"],
        "split_ms": {k: round(v, 4) for k, v in prim["kernel_ms"].items()},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": kd["achieved"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": kd["frac"],
                     "traffic": load_traffic(args.workload, args.causal, dom),
                     "flop_per_launch": kd["flop_per_launch"],
                     "avg_launch_ms": kd["avg_launch_ms"]},
        "kernels": prim["kernels"],
        "forward": prim["forward"],
        "recompute_L": prim["recompute_L"],
        "forward_backward": prim["forward_backward"],
    }
    if len(results) > 1:
        other = results[not args.causal]
        line["causal" if not args.causal else "non_causal"] = {
            "value": round(other["tflops"], 3), "ms_per_step": round(other["ms_per_step"], 4),
            "step_ms": other["step_ms"],
            "pct_bf16_peak": round(other["pct_peak"], 2),
            "split_ms": {k: round(v, 4) for k, v in other["kernel_ms"].items()},
            "kernels": other["kernels"], "forward": other["forward"],
            "recompute_L": other["recompute_L"], "forward_backward": other["forward_backward"]}
    if not (args.no_extra or args.no_other) and args.workload == "h32_n8192_d128_bf16":
        # the two other full-size workloads (their own causal modes), the
        # same timed step; context beside the line, not its value
        line["other_workloads"] = [other_workload(si.WORKLOADS[n], args)
                                   for n in ("b4_h16_n4000_d128_bf16_q4", "h8_n32768_d128_bf16")]
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.causal, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
