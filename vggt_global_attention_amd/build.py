"""Build libvggtattn.so (gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvggtattn.so")
# The same sources with the tuning overrides compiled in (environment
# variables that force tile, split and GEMM choices; see csrc/plan.h): for
# sweeps and for the tests that force a choice.  Never the product library.
TUNE_LIB = os.path.join(PKG, "libvggtattn_tune.so")
# Host code (argument checks, planning, the schedule driver) built with
# AddressSanitizer and UndefinedBehaviorSanitizer, device code unchanged: for
# the CPU-side ABI tests only (tests/test_host_sanitizers.py).
SAN_LIB = os.path.join(PKG, "libvggtattn_san.so")
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SOURCES = ["api.cpp", "prep.hip", "gemm.hip", "attention.hip", "subsample.hip",
           "desc.hip", "schedule.cpp", "static_scratch.hip", "merge.hip"]

# Packed fp32 VALU ops are kept out of every kernel on purpose.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, extra_flags=(), tuning: bool = True) -> str:
    """Compile every HIP source for gfx950 and link the shared library (and,
    unless tuning=False, the tuning build beside it)."""
    if tuning:
        _link(TUNE_LIB, verbose, (*extra_flags, "-DVGGT_ATTN_TUNING"))
    return _link(LIB, verbose, extra_flags)


def build_sanitized(verbose: bool = False) -> str:
    """The host-sanitizer build (SAN_LIB); load it only in a process that
    preloads the compiler's ASan runtime."""
    return _link(SAN_LIB, verbose, SAN_FLAGS)


def _link(out: str, verbose: bool, extra_flags) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-shared", "-I", INCLUDE, "-I", CSRC,
           "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
