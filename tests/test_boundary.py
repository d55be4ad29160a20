"""CPU-only checks of the C ABI boundary: the library loads, exports every
symbol include/fa_bwd.h declares, and rejects bad arguments before touching a
device.  Also checks that the oracle and the GPU path share no code."""
import ctypes
import os
import re

import pytest

import attention_fa_bwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_bwd.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    names = _declared()
    assert {"fa_fwd_lse", "fa_lse", "fa_bwd_preprocess", "fa_bwd", "fa_bwd_convert_dq",
            "fa_bwd_dkdv", "fa_bwd_dq", "fa_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_has_same_names():
    for n in _declared():
        if n != "fa_last_hip_error":   # read by the binding's error path, not exposed
            assert callable(getattr(fa, n)), n


def test_strerror():
    for code in (0, 1, 2, 3, 99):
        s = fa.fa_strerror(code)
        assert isinstance(s, str) and s


ALIGNED = 4096   # a non-null, 16-byte aligned address that is never dereferenced


def _bwd(lib, **kw):
    a = dict(dtype=1, ptr=ALIGNED, B=1, H=1, N=8, d=64)
    a.update(kw)
    p = a["ptr"]
    return lib.fa_bwd(a["dtype"], p, p, p, p, p, p, p, p, p, a["B"], a["H"], a["N"], a["d"],
                      0.125, 0, None)


def test_invalid_arguments_rejected_before_device_work():
    lib = fa.load()
    assert _bwd(lib, ptr=None) == fa.FA_EINVAL
    assert _bwd(lib, ptr=ALIGNED + 4) == fa.FA_EINVAL        # misaligned
    assert _bwd(lib, B=0) == fa.FA_EINVAL
    assert _bwd(lib, N=-3) == fa.FA_EINVAL
    assert _bwd(lib, dtype=7) == fa.FA_EINVAL
    assert _bwd(lib, B=70000) == fa.FA_EINVAL
    assert _bwd(lib, B=60000, H=60000, N=60000, d=128) == fa.FA_EINVAL   # > 2^40 elements
    assert _bwd(lib, N=(1 << 30) + 1, d=16) == fa.FA_EINVAL              # N beyond 32-bit tile indices
    assert _bwd(lib, N=2**31 - 1, d=16) == fa.FA_EINVAL
    p = ALIGNED
    assert lib.fa_fwd_lse(1, p, p, None, p, p, 1, 1, 8, 64, 0.1, 0, None) == fa.FA_EINVAL
    assert lib.fa_lse(1, p, p, None, 1, 1, 8, 64, 0.1, 0, None) == fa.FA_EINVAL
    assert lib.fa_lse(2, p, p + 8, p, 1, 1, 8, 128, 0.1, 0, None) == fa.FA_EINVAL   # misaligned
    assert lib.fa_lse(5, p, p, p, 1, 1, 8, 128, 0.1, 0, None) == fa.FA_EINVAL
    # the softmax scale must be finite and positive for the attention calls
    for bad in (0.0, -0.125, float("nan"), float("inf")):
        assert lib.fa_fwd_lse(1, p, p, p, p, p, 1, 1, 8, 128, bad, 0, None) == fa.FA_EINVAL
        assert lib.fa_lse(1, p, p, p, 1, 1, 8, 64, bad, 1, None) == fa.FA_EINVAL
        assert lib.fa_bwd(1, p, p, p, p, p, p, p, p, p, 1, 1, 8, 64, bad, 0, None) == fa.FA_EINVAL
        assert lib.fa_bwd_dkdv(1, p, p, p, p, p, p, p, p, 1, 1, 8, 128, bad, 0, None) == fa.FA_EINVAL
        assert lib.fa_bwd_dq(2, p, p, p, p, p, p, p, 1, 1, 8, 128, bad, 1, None) == fa.FA_EINVAL
    assert lib.fa_bwd_preprocess(1, p, p, None, 1, 1, 8, 64, None) == fa.FA_EINVAL
    assert lib.fa_bwd_convert_dq(0, None, p, 1, 1, 8, 64, 0.1, None) == fa.FA_EINVAL


@pytest.mark.parametrize("d", [8, 48, 96, 256])
def test_unsupported_head_dim(d):
    lib = fa.load()
    p = ALIGNED
    assert _bwd(lib, d=d) == fa.FA_EUNSUPPORTED
    assert lib.fa_fwd_lse(0, p, p, p, p, p, 1, 1, 8, d, 0.1, 1, None) == fa.FA_EUNSUPPORTED
    assert lib.fa_lse(1, p, p, p, 1, 1, 8, d, 0.1, 1, None) == fa.FA_EUNSUPPORTED
    assert lib.fa_bwd_preprocess(1, p, p, p, 1, 1, 8, d, None) == fa.FA_EUNSUPPORTED
    assert lib.fa_bwd_convert_dq(1, p, p, 1, 1, 8, d, 0.1, None) == fa.FA_EUNSUPPORTED


def test_noalloc_validates_arguments_and_size():
    """fa_bwd_noalloc checks its arguments like fa_bwd and refuses problems
    whose D does not fit its static scratch array (FA_ESCRATCH), before any
    device work."""
    lib = fa.load()
    p = ALIGNED
    call = lambda dtype=1, q=p, B=1, H=1, N=8, d=64, sc=0.125: lib.fa_bwd_noalloc(
        dtype, q, p, p, p, p, p, p, p, p, B, H, N, d, sc, 0, None)
    assert call(q=None) == fa.FA_EINVAL
    assert call(q=p + 4) == fa.FA_EINVAL
    assert call(dtype=9) == fa.FA_EINVAL
    assert call(sc=0.0) == fa.FA_EINVAL
    assert call(d=96) == fa.FA_EUNSUPPORTED
    rows = fa.FA_NOALLOC_MAX_ROWS
    assert call(B=1, H=4, N=rows // 4 + 1, d=16) == fa.FA_ESCRATCH
    assert call(B=2, H=64, N=32768 + 1, d=128) == fa.FA_ESCRATCH
    assert "FA_NOALLOC_MAX_ROWS" in fa.fa_strerror(fa.FA_ESCRATCH)


def test_split_passes_validate_arguments():
    lib = fa.load()
    p = ALIGNED
    assert _bwd(lib, dtype=3) == fa.FA_EINVAL
    assert lib.fa_bwd_dkdv(1, p, None, p, p, p, p, p, p, 1, 1, 8, 128, 0.1, 0, None) == fa.FA_EINVAL
    assert lib.fa_bwd_dq(1, p, p, p, p, p, p, None, 1, 1, 8, 128, 0.1, 0, None) == fa.FA_EINVAL
    assert lib.fa_bwd_dkdv(2, p, None, p, p, p, p, p, p, 1, 1, 8, 64, 0.1, 0, None) == fa.FA_EINVAL
    assert lib.fa_bwd_dq(0, p, p, p, p, p, p, p, 1, 1, 8, 96, 0.1, 1, None) == fa.FA_EUNSUPPORTED
    assert lib.fa_bwd_dkdv(0, p, p, p, p, p, p, p, p, 1, 1, 8, 8, 0.1, 1, None) == fa.FA_EUNSUPPORTED


# Run in a child process: every entry point with valid arguments must return
# FA_EHIP (and never crash) when no device is present.  The child first asks
# the HIP runtime how many devices it sees and makes no call at all if there
# is one, so the fake addresses below never reach a kernel.
_NO_DEVICE_CHILD = r"""
import ctypes, ctypes.util, json, sys
lib = ctypes.CDLL(sys.argv[1])
name = ctypes.util.find_library("amdhip64") or "/opt/rocm/lib/libamdhip64.so"
hip = ctypes.CDLL(name)
n = ctypes.c_int(0)
rc = hip.hipGetDeviceCount(ctypes.byref(n))
if rc == 0 and n.value > 0:
    print(json.dumps({"device": True}))
    sys.exit(0)
p, f = ctypes.c_void_p(4096), ctypes.c_float
lib.fa_last_hip_error.restype = ctypes.c_int
out = {"device": False, "count_rc": rc}
calls = {
    "fa_fwd_lse": lambda d, t: lib.fa_fwd_lse(t, p, p, p, p, p, 1, 2, 40, d, f(0.125), 1, None),
    "fa_lse": lambda d, t: lib.fa_lse(t, p, p, p, 1, 2, 40, d, f(0.125), 0, None),
    "fa_bwd_preprocess": lambda d, t: lib.fa_bwd_preprocess(t, p, p, p, 1, 2, 40, d, None),
    "fa_bwd": lambda d, t: lib.fa_bwd(t, p, p, p, p, p, p, p, p, p, 1, 2, 40, d, f(0.125), 1, None),
    "fa_bwd_dkdv": lambda d, t: lib.fa_bwd_dkdv(t, p, p, p, p, p, p, p, p, 1, 2, 40, d, f(0.125), 0, None),
    "fa_bwd_dq": lambda d, t: lib.fa_bwd_dq(t, p, p, p, p, p, p, p, 1, 2, 40, d, f(0.125), 1, None),
    "fa_bwd_convert_dq": lambda d, t: lib.fa_bwd_convert_dq(t, p, p, 1, 2, 40, d, f(0.125), None),
    "fa_bwd_noalloc": lambda d, t: lib.fa_bwd_noalloc(t, p, p, p, p, p, p, p, p, p, 1, 2, 40, d, f(0.125), 1, None),
}
for nm, call in calls.items():
    for d in (16, 32, 64, 128):
        for t in (0, 1, 2):
            out[f"{nm}/d{d}/t{t}"] = [call(d, t), lib.fa_last_hip_error()]
print(json.dumps(out))
"""


def test_every_entry_point_reports_no_device():
    """Without a device every entry point returns FA_EHIP with the HIP error
    recorded, for every dtype and head dim, before any launch."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", _NO_DEVICE_CHILD, fa.lib_path()],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout.strip().splitlines()[-1])
    if out["device"]:
        pytest.skip("a device is present; the no-device path cannot be exercised here")
    results = {k: v for k, v in out.items() if "/" in k}
    assert len(results) == 8 * 4 * 3
    for k, (rc, hip_err) in results.items():
        assert rc == fa.FA_EHIP, (k, rc)
        assert hip_err != 0, k


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        fa.forward(x, x, x, 0.25, False)


def test_binding_checks_every_shape_before_the_library():
    """The C-ABI sees only pointers and (B, H, N, d): a smaller tensor would be
    read or written out of bounds, so the binding compares every shape with the
    one the sizes imply first."""
    import torch
    B, H, N, d = 1, 2, 8, 16
    x4 = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    f3 = torch.zeros(B, H, N)
    f4 = torch.zeros(B, H, N, d)
    short = torch.zeros(B, H, N - 1, d, dtype=torch.bfloat16)
    bad3 = torch.zeros(B, H, N + 1)
    bad4 = torch.zeros(B, H, N, d + 1)
    cases = [
        lambda: fa.fa_fwd_lse(x4, short, x4, x4, f3, 0.25, False),
        lambda: fa.fa_fwd_lse(x4, x4, x4, x4, bad3, 0.25, False),
        lambda: fa.fa_lse(x4, short, f3, 0.25, True),
        lambda: fa.fa_bwd_preprocess(x4, short, f3),
        lambda: fa.fa_bwd_preprocess(x4, x4, bad3),
        lambda: fa.fa_bwd(x4, x4, short, x4, f3, f3, f4, x4, x4, 0.25, False),
        lambda: fa.fa_bwd(x4, x4, x4, x4, f3, bad3, f4, x4, x4, 0.25, False),
        lambda: fa.fa_bwd(x4, x4, x4, x4, f3, f3, f4, x4, short, 0.25, False),
        lambda: fa.fa_bwd_dkdv(x4, x4, x4, short, f3, f3, x4, x4, 0.25, True),
        lambda: fa.fa_bwd_dq(x4, x4, x4, x4, f3, f3, bad4, 0.25, True),
        lambda: fa.fa_bwd_convert_dq(bad4, x4, 0.25),
    ]
    for i, call in enumerate(cases):
        with pytest.raises(ValueError, match="expected shape"):
            call()


def _sources(*dirs, exts=(".py", ".hip", ".hpp", ".h", ".c", ".cpp")):
    for d in dirs:
        for base, _, files in os.walk(os.path.join(ROOT, d)):
            for f in files:
                if f.endswith(exts):
                    yield os.path.join(base, f)


def test_oracle_and_gpu_path_share_no_code():
    for f in _sources("oracle"):
        t = open(f, encoding="utf-8").read()
        assert "attention_fa_bwd_amd" not in t and "fa_bwd.h" not in t, f
    for f in _sources("attention_fa_bwd_amd", "include"):
        t = open(f, encoding="utf-8").read()
        assert not re.search(r"\boracle\b", t), f
