"""Seeded synthetic inputs, shared by the tests, the smoke check and the benchmark.

This module only draws random numbers; it holds none of the attention
arithmetic.  Every tensor comes from its own CPU ``torch.Generator`` seeded with
``1000 * workload.cid + tensor_index`` so the GPU path and the fp64 oracle see
the same bytes.

Value recipe ("N(0, s)" is read as variance s):
  X ~ N(0, 1); Wqkv, Wo ~ N(0, 1/d); gamma = 1 + N(0, 0.1); beta ~ N(0, 0.1)
  (independent per head and feature, for q and for k).  X, Wqkv and Wo are
  rounded to bf16 (round to nearest even); gamma and beta stay fp32.
  Workloads with duplicated frames then pick ``dup_frames`` frame indices in
  1..S-1 without replacement and, in increasing order, set
  X[s] = bf16(X[s-1] + N(0, 0.05)), a temporally redundant video.
"""

from __future__ import annotations

import math

import torch

from .configs import Workload

TENSOR_ORDER = ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta",
                "dup_pick", "dup_noise")


def _gen(w: Workload, name: str) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * w.cid + TENSOR_ORDER.index(name))
    return g


def _normal(shape, std, g, dtype=torch.float32):
    return torch.randn(shape, generator=g, dtype=torch.float32).mul_(std).to(dtype)


def make_inputs(w: Workload, fp32: bool = False) -> dict:
    """Draw one workload's inputs as CPU tensors.

    ``fp32=True`` returns the same draws without the bf16 rounding (oracle-only
    variant).  Returned keys: X [S,T,d], Wqkv [3d,d], Wo [d,d] (bf16 unless
    fp32), q_gamma/q_beta/k_gamma/k_beta [H,Dh] fp32.
    """
    d, H, Dh = w.d, w.H, w.Dh
    wdt = torch.float32 if fp32 else torch.bfloat16
    out = {}
    X = _normal((w.S, w.T, d), 1.0, _gen(w, "X"))
    out["Wqkv"] = _normal((3 * d, d), 1.0 / math.sqrt(d), _gen(w, "Wqkv"), wdt)
    out["Wo"] = _normal((d, d), 1.0 / math.sqrt(d), _gen(w, "Wo"), wdt)
    sd = math.sqrt(0.1)
    out["q_gamma"] = 1.0 + _normal((H, Dh), sd, _gen(w, "q_gamma"))
    out["q_beta"] = _normal((H, Dh), sd, _gen(w, "q_beta"))
    out["k_gamma"] = 1.0 + _normal((H, Dh), sd, _gen(w, "k_gamma"))
    out["k_beta"] = _normal((H, Dh), sd, _gen(w, "k_beta"))
    X = X.to(wdt)
    if w.dup_frames:
        pick = torch.randperm(w.S - 1, generator=_gen(w, "dup_pick"))[: w.dup_frames] + 1
        pick, _ = torch.sort(pick)
        gn = _gen(w, "dup_noise")
        for s in pick.tolist():
            noise = _normal((w.T, d), math.sqrt(0.05), gn)
            X[s] = (X[s - 1].float() + noise).to(wdt)
        out["dup_frames"] = pick
    out["X"] = X
    return out


BLOCK_TENSORS = ("Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta", "layer_scale")


def make_block_weights(w: Workload, n_blocks: int, ls: float = 1e-5) -> list:
    """Weights of `n_blocks` blocks for a layer schedule, as CPU tensors.

    Block b, tensor i draws from its own generator seeded with
    10_000_000 + 1000 * cid + 10 * b + i (b < 100).  Same value recipe as
    make_inputs; the LayerScale vector is ls * (1 + N(0, 0.01)) per channel,
    fp32.  Returns a list of dicts with the keys of BLOCK_TENSORS.
    """
    if n_blocks > 100:
        raise ValueError("at most 100 blocks")
    d, H, Dh = w.d, w.H, w.Dh
    sd = math.sqrt(0.1)
    out = []
    for b in range(n_blocks):
        def gen(name):
            g = torch.Generator(device="cpu")
            g.manual_seed(10_000_000 + 1000 * w.cid + 10 * b + BLOCK_TENSORS.index(name))
            return g
        out.append({
            "Wqkv": _normal((3 * d, d), 1.0 / math.sqrt(d), gen("Wqkv"), torch.bfloat16),
            "Wo": _normal((d, d), 1.0 / math.sqrt(d), gen("Wo"), torch.bfloat16),
            "q_gamma": 1.0 + _normal((H, Dh), sd, gen("q_gamma")),
            "q_beta": _normal((H, Dh), sd, gen("q_beta")),
            "k_gamma": 1.0 + _normal((H, Dh), sd, gen("k_gamma")),
            "k_beta": _normal((H, Dh), sd, gen("k_beta")),
            "layer_scale": ls * (1.0 + _normal((d,), 0.1, gen("layer_scale"))),
        })
    return out


def make_descriptors(w: Workload, M: int, salt: int = 0, scale: float = 1.0) -> torch.Tensor:
    """M descriptor tokens [M, d], bf16: scale * N(0, 1), the value recipe of X
    (descriptors are token states of the model's width).  Seed
    20_000_000 + 1000 * cid + salt."""
    g = torch.Generator(device="cpu")
    g.manual_seed(20_000_000 + 1000 * w.cid + salt)
    return _normal((M, w.d), scale, g).to(torch.bfloat16)


def sample_rows(w: Workload, n_rows: int, seed: int = 7) -> torch.Tensor:
    """A seeded sample of flat row indices (s*T + t) for row-sampled parity.

    Always includes all 17 special tokens of the first and last frame and the
    last patch token of every sampled frame boundary; the rest is uniform.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * w.cid + 500 + seed)
    fixed = [t for t in range(17)] + [(w.S - 1) * w.T + t for t in range(17)]
    fixed += [w.T - 1, w.N - 1]
    rnd = torch.randint(0, w.N, (max(0, n_rows - len(fixed)),), generator=g).tolist()
    rows = sorted(set(fixed + rnd))
    return torch.tensor(rows, dtype=torch.int64)
