"""Host-side checks of the decode plan: the split planning and the index
math that the decode and merge kernels share (csrc/decode_plan.h,
csrc/oscar_internal.h) are compiled for the host and run on random batches
(every page and window covered exactly once, indices inside each pair, the
launch order a permutation of the batch, blocks writing the output rows
themselves exactly when no pair is split).  No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_decode_plan_covers_every_page_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "decode_plan_check"
    src = os.path.join(ROOT, "tests", "csrc", "decode_plan_check.cpp")
    inc = os.path.join(ROOT, "bit_kv_cache_segment_amd", "csrc")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I", inc, src,
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe), "3000"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "decode plan ok" in r.stdout
