"""bench.py end to end on the GPU: the one JSON line it prints for a small
workload carries every field of its contract (metric, value, unit, the step
count and warm-up it was given, the roofline of the dominant kernel, the
per-call split) with values that agree with each other."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REQUIRED = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
            "roofline", "cpu_baseline")


def test_bench_line_contract():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "7", "--warmup", "2",
           "--no-cpu", "--no-extra", "--workload", "h8_n1024_d64_bf16"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in REQUIRED:
        assert k in d, k
    assert d["steps"] == 7 and d["warmup"] == 2 and d["n_gpus"] == 1
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["vs_baseline"] is None and d["cpu_baseline"] is None   # --no-cpu
    cfg = d["config"]
    assert (cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]) == (1, 8, 1024, 64, False)
    # value is the workload's FLOPs over the timed steps' mean
    flops = 10.0 * 1 * 8 * 1024 * 1024 * 64
    assert d["value"] == pytest.approx(flops / (d["ms_per_step"] * 1e-3) / 1e12, rel=5e-3)
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == pytest.approx(2516.6)
    assert 0.0 < rf["frac"] < 1.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=3e-3)
    assert rf["achieved"] == pytest.approx(rf["flop_per_launch"] / (rf["avg_launch_ms"] * 1e-3) / 1e12,
                                           rel=1e-3)
    # every call of the step is in the split, and the dominant kernel is fa_bwd
    assert set(d["split_ms"]) == {"fa_bwd_preprocess", "fa_bwd", "fa_bwd_convert_dq"}
    assert rf["kernel"] == "fa_bwd"
    assert rf["avg_launch_ms"] == pytest.approx(d["split_ms"]["fa_bwd"], rel=1e-3)
