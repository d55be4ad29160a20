"""Host-side logic of bench.py: the one-GPU contract and the traffic record
lookup (no GPU needed)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_matches_current_kernels():
    """The committed HBM-traffic record carries the hash of the kernel
    sources it was measured on; bench.py reports it only while they match."""
    rec = json.load(open(bench.TRAFFIC_FILE))
    for key in ("fa_bwd_dkdv/h32_n8192_d128_bf16_full", "fa_bwd_dq/h32_n8192_d128_bf16_full"):
        assert key in rec["entries"]
    if rec["kernel_source_hash"] == bench.kernel_source_hash():
        assert bench.load_traffic("h32_n8192_d128_bf16", False, "fa_bwd_dkdv") > 0
    else:
        assert bench.load_traffic("h32_n8192_d128_bf16", False, "fa_bwd_dkdv") is None
