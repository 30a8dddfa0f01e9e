"""The multiply-shift division of the kernels' row maps and block coordinates.

`fast_div` / `fdiv` (csrc/common.h) replace integer division by a run-time
divisor with one multiply and a shift; the attention kernel's block
coordinates and the projection kernels' row maps depend on it being exact for
every numerator below 2^31.  tests/native/fast_div_check.hip calls the same
header functions on the host (no GPU: host-only compile) over edge cases and a
seeded sample of 4 M (n, d) pairs against C++ integer division.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_fast_div_is_exact():
    src = os.path.join(ROOT, "tests", "native", "fast_div_check.hip")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "fast_div_check")
        build = subprocess.run(
            [HIPCC, "--cuda-host-only", "-O2", "-std=c++17",
             "-I", os.path.join(ROOT, "vggt_global_attention_amd", "csrc"),
             "-I", os.path.join(ROOT, "include"), "-x", "hip", src, "-o", exe],
            capture_output=True, text=True, timeout=300)
        assert build.returncode == 0, build.stderr[-2000:]
        run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:]
    assert " 0 failures" in run.stdout, run.stdout
