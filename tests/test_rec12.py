"""The 12-bit block floating-point records of the selection partials, checked on the host.

The selection kernels store each (row, slot, head) partial's value sum as 128 signed 12-bit
integers with one power-of-two step, and fold the step into the partial's (max, sum) pair so the
merge weights stay exact.  tests/rec12_check.hip calls the same encode / decode functions the
kernels call (fast_common.hpp, host and device) and checks: the bit layout of a pack, rounding
to nearest with ties to even, the exponent rule (no integer beyond +-2047, clamps), the step
bound of every decoded value over magnitudes from 1e-12 to 1e20 (zeros, exact powers of two,
maxima just below a power of two), and that merging records through the folded (max, sum)
pairs equals the merge of the exact partials within the records' step bound.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_rec12_records(tmp_path):
    exe = tmp_path / "rec12_check"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "rec12_check.hip"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "rec12 ok" in r.stdout, r.stdout[-3000:] + r.stderr[-2000:]
