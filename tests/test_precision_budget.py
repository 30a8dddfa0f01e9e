"""Precision budget of the attention path: which 16-bit rounding points a
kernel can afford under the bar relL1 <= 2e-3 against the fp64 definition.

A CPU emulation (fp64 arithmetic, explicit rounding to fp16 or bf16 at the
points a flash-style kernel stores values: q and k after LayerNorm + RoPE, v,
the unnormalised probabilities P, the normalised output O before Wo, and Y)
of one global block at the model's shape (d = 1024, 16 heads of 64, 26 x 39
patches), compared with the oracle.  It fixes the library's precision design:
fp16 for q, k, v, P and O with bf16 at the boundary fits the bar, a plain
bf16 pipeline does not.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.vggt_oracle import _project
from test_oracle_pins import small_case


def fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).to(
        torch.float64).numpy()


def ident(x):
    return x


def emulate(X, p, rq, rk, rv, rP, rO, rY):
    """Global block with rounding at the stored points; softmax per row is
    exact fp64 apart from the rounding of the unnormalised P."""
    S, T, d = X.shape
    Xf = X.reshape(S * T, d)
    t = np.tile(np.arange(T), S)
    f = _project(Xf, t, p)
    q, k, v = rq(f["q"]), rk(f["k"]), rv(f["v"])
    O = np.empty((S * T, p.H, p.Dh))
    for h in range(p.H):
        a = (q[:, h] @ k[:, h].T) / math.sqrt(p.Dh)
        P = rP(np.exp(a - a.max(axis=1, keepdims=True)))
        O[:, h] = (P @ v[:, h]) / P.sum(axis=1, keepdims=True)
    Y = rO(O.reshape(S * T, d)) @ p.Wo.T
    return rY(Y).reshape(S, T, d)


@pytest.fixture(scope="module")
def case():
    X, p = small_case(S=2, gh=26, gw=39, d=1024, H=16, seed=41, gscale=0.3, bscale=0.3)
    X = bf16(X)
    p.Wqkv = bf16(p.Wqkv)
    p.Wo = bf16(p.Wo)
    ref = oracle.global_attention(X, p, threads=4)
    return X, p, ref


def rel_l1(y, ref):
    return float(np.abs(y - ref).sum() / np.abs(ref).sum())


def test_no_rounding_is_the_definition(case):
    X, p, ref = case
    y = emulate(X, p, ident, ident, ident, ident, ident, ident)
    assert rel_l1(y, ref) < 1e-12


def test_library_design_fits_the_bar(case):
    X, p, ref = case
    only_y = rel_l1(emulate(X, p, ident, ident, ident, ident, ident, bf16), ref)
    design = rel_l1(emulate(X, p, fp16, fp16, fp16, fp16, fp16, bf16), ref)
    plain_bf16 = rel_l1(emulate(X, p, bf16, bf16, bf16, bf16, bf16, bf16), ref)
    # bf16 output rounding alone costs most of the budget ...
    assert 1.0e-3 < only_y < 1.8e-3, only_y
    # ... fp16 inside adds little and stays under the bar ...
    assert design < 2e-3 and design < 1.25 * only_y, (design, only_y)
    # ... while a plain bf16 pipeline does not fit.
    assert plain_bf16 > 2e-3, plain_bf16
