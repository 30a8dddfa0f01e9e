"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host side -- argument checks, workspace planning, the layer
schedule driver, the descriptor cache and status entry points -- is built
with -fsanitize=address,undefined on the host only (build.build_sanitized)
and the CPU ABI tests (tests/test_abi.py, which make no GPU call) run against
it in a child process that preloads the compiler's ASan runtime; any report
aborts the child (halt_on_error).  No GPU is involved."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

from vggt_global_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, %(root)r)
sys.path.insert(0, %(tests)r)
from vggt_global_attention_amd import binding as B
B.lib(%(lib)r)
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", %(abi)r]))
"""


def _asan_runtime():
    clang = "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def test_abi_under_host_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("the ROCm clang ASan runtime is not installed")
    lib = build.build_sanitized()
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = CHILD % {"root": ROOT, "tests": os.path.join(ROOT, "tests"), "lib": lib,
                    "abi": os.path.join(ROOT, "tests", "test_abi.py")}
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
