"""GPU-side helpers for the parity tests: move seeded inputs to the device and
run the library through its C ABI (via the torch front end)."""

from __future__ import annotations

import contextlib
import sys

import numpy as np
import pytest
import torch

from vggt_global_attention_amd import api
from vggt_global_attention_amd import binding as B

KEYS = ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.lib()  # raises if the HIP library is missing: no fallback exists


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(inp: dict, dev="cuda") -> dict:
    return {k: inp[k].to(dev).contiguous() for k in KEYS}


def run(mode: str, w, d: dict, X=None, Y=None, **shape_kw) -> torch.Tensor:
    X = d["X"] if X is None else X
    blk = api.Block(mode, X, w.H, w.grid_h, w.grid_w, **shape_kw)
    out = blk(X, d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"], d["k_gamma"], d["k_beta"], Y=Y)
    torch.cuda.synchronize()
    return out


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


@contextlib.contextmanager
def tuned(monkeypatch, **knobs):
    """Run the block through the tuning build with the given overrides set
    (e.g. VGGT_ATTN_SPLIT=1); the product library reads no environment."""
    for k, v in knobs.items():
        monkeypatch.setenv(k, str(v))
    try:
        with B.tuning_build():
            yield
    finally:
        for k in knobs:
            monkeypatch.delenv(k, raising=False)
