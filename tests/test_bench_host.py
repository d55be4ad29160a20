"""Host-side logic of bench.py: the one-GPU contract, the choice of timed
configurations for every --workload, the FLOP and byte models, and the traffic
record lookup (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

import bench
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_default_run_times_every_config():
    args = bench.parse([])
    assert not args.reference_gemm and bench.parse(["--reference-gemm"]).reference_gemm
    runs = bench.plan(args)
    assert runs[0] == ("h32_n8192_d128_bf16", False)
    assert sorted(runs) == sorted(bench.CONFIGS)
    assert len(set(runs)) == 7
    # every workload, in every causal mode it is specified for
    for name, wl in si.WORKLOADS.items():
        for c in wl.causal:
            assert (name, c) in runs


@pytest.mark.parametrize("name", sorted(si.WORKLOADS))
def test_every_workload_choice_plans(name):
    wl = si.WORKLOADS[name]
    for c in wl.causal:
        argv = ["--workload", name] + (["--causal"] if c else [])
        assert bench.plan(bench.parse(argv + ["--no-extra"])) == [(name, c)]
        runs = bench.plan(bench.parse(argv))
        assert runs[0] == (name, c) and sorted(runs) == sorted(bench.CONFIGS)
        other = bench.plan(bench.parse(argv + ["--no-other"]))
        assert other[0] == (name, c) and sorted(other) == sorted((name, m) for m in wl.causal)
        # the library supports the workload's dtype and head dim on both passes
        assert wl.d in (16, 32, 64, 128) and wl.dtype in ("fp32", "bf16", "fp16")
    missing = [m for m in (False, True) if m not in wl.causal]
    for c in missing:
        with pytest.raises(SystemExit):
            bench.plan(bench.parse(["--workload", name] + (["--causal"] if c else [])))


def test_flop_and_byte_models():
    wl = si.WORKLOADS["h32_n8192_d128_bf16"]
    f = wl.flops(False)
    assert f == 10 * 32 * 8192 ** 2 * 128 and wl.flops(True) == f / 2
    # algorithmic: the five products, split 8 : 2 between the passes
    assert bench.pass_flops(wl, False, "fa_bwd") == f
    assert bench.pass_flops(wl, False, "fa_bwd_dkdv") == 0.8 * f
    assert bench.pass_flops(wl, True, "fa_bwd") == 0.5 * f
    assert bench.pass_flops(wl, True, "fa_bwd_dq") == 0.1 * f
    assert (bench.pass_flops(wl, False, "fa_bwd_dkdv") + bench.pass_flops(wl, False, "fa_bwd_dq")
            == bench.pass_flops(wl, False, "fa_bwd"))
    # executed: the dQ pass forms S and dP again
    assert bench.pass_flops(wl, False, "fa_bwd", executed=True) == 1.4 * f
    assert bench.pass_flops(wl, True, "fa_bwd_dq", executed=True) == 0.3 * f
    r = bench.kernel_rates(wl, False, "fa_bwd", 2.0, bench.PEAK_BF16_TFLOPS)
    assert r["frac"] == round(f / 2e-3 / 1e12 / bench.PEAK_BF16_TFLOPS, 4)
    assert abs(r["executed_frac"] - 1.4 * r["frac"]) < 1e-3
    rows = 32 * 8192
    b = bench.hbm_kernel_bytes(wl)
    assert b["fa_bwd_preprocess"] == rows * 128 * 4 + rows * 4
    assert b["fa_bwd_convert_dq"] == rows * 128 * 6
    c1 = si.WORKLOADS["n48_d16_fp32"]
    assert bench.hbm_kernel_bytes(c1)["fa_bwd_convert_dq"] == 48 * 16 * 8
    assert bench.compute_peak(c1) == ("alu", bench.PEAK_FP32_VALU_TFLOPS)
    assert bench.compute_peak(wl) == ("mfma", bench.PEAK_BF16_TFLOPS)


def test_traffic_record_matches_current_kernels():
    """The committed HBM-traffic record carries the hash of the kernel
    sources it was measured on; bench.py reports it only while they match."""
    rec = json.load(open(bench.TRAFFIC_FILE))
    for key in ("fa_bwd/h32_n8192_d128_bf16_full", "fa_bwd/h32_n8192_d128_bf16_causal"):
        assert key in rec["entries"]
    if rec["kernel_source_hash"] == bench.kernel_source_hash():
        assert bench.load_traffic("h32_n8192_d128_bf16", False, "fa_bwd") > 0
    else:
        assert bench.load_traffic("h32_n8192_d128_bf16", False, "fa_bwd") is None
