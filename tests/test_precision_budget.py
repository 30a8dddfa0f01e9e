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


def test_bf16_operand_variant_bar(case):
    """The bf16-operand variant rounds q, k, v, P, O (and Y) to bf16: its bar
    (helpers.BF16OPS_*) sits a third or more above what that rounding costs."""
    from helpers import BF16OPS_MAX, BF16OPS_MEAN, BF16OPS_RELL1, metrics
    X, p, ref = case
    m = metrics(emulate(X, p, bf16, bf16, bf16, bf16, bf16, bf16), ref)
    assert 3e-3 < m["relL1"] < BF16OPS_RELL1 / 1.3, m
    assert m["max_over_max"] < BF16OPS_MAX / 1.3, m
    assert m["mean_over_max"] < BF16OPS_MEAN / 1.3, m


# ----------------------------------------------------------------------------
# The attention kernel's softmax reference rule, emulated on the CPU
# ----------------------------------------------------------------------------
# The kernel takes logits in base 2 (q carries log2(e)/sqrt(Dh)) relative to a
# per-row reference m and rounds P = 2^(s - m) to fp16.  It knows an upper
# bound of every logit of a row before the first 64-key tile: |q| * max|k|
# (Cauchy-Schwarz), times 1 + 2^-10.  After the first tile a row whose max m0
# satisfies bound - m0 <= SETTLE_GAP is "settled": its reference is pinned at
# max(m0, bound - PIN_BELOW) and never moves again (no logit can push P past
# 2^PIN_BELOW).  Other rows keep an online max -- the exact running max over
# the first EAGER_TILES tiles, later lazy rescaling (only when a tile's max
# exceeds m + TAU) -- and re-check the settle condition per tile.  The pinned
# reference can sit up to SETTLE_GAP - PIN_BELOW above the row's true max,
# which pushes the row's probabilities toward fp16's subnormal range.
TAU, PIN_BELOW, SETTLE_GAP, EAGER_TILES = 8.0, 15.0, 19.0, 16
LOG2E = 1.0 / math.log(2.0)


def _ln(x, g, b):
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(var + 1e-5) * g + b


def kernel_softmax_core(q, k, v, settle_gap=SETTLE_GAP, tile=64):
    """Emulated attention core of one head: q [R,64] (scaled, fp16 values),
    k, v [N,64] (fp16 values).  Returns (O rounded to fp16, settled flags)."""
    R, N = q.shape[0], k.shape[0]
    kmax = np.sqrt((k * k).sum(1)).max()
    bound = np.sqrt((q * q).sum(1)) * kmax * (1 + 2.0 ** -10)
    m = np.zeros(R)
    l = np.zeros(R)
    O = np.zeros((R, q.shape[1]))
    settled = np.zeros(R, bool)
    for t0 in range(0, N, tile):
        s = q @ k[t0:t0 + tile].T - m[:, None]
        first = t0 == 0
        track = first | ~settled  # per row (the kernel tracks per wave: never less precise)
        mt = s.max(1)
        lazy = 0.0 if t0 < EAGER_TILES * tile else TAU
        mn = np.where(first | (mt > lazy), m + mt, m)
        ok = mn >= bound - settle_gap
        mn = np.where(ok, np.maximum(mn, bound - PIN_BELOW), mn)
        mn = np.where(track, mn, m)
        settled |= track & ok
        dl = mn - m
        s -= dl[:, None]
        if not first:
            al = np.exp2(-dl)
            l *= al
            O *= al[:, None]
        m = mn
        P = fp16(np.exp2(s))
        l += P.sum(1)
        O += P @ v[t0:t0 + tile]
    return fp16(O / l[:, None]), settled


def _exact_core(q, k, v):
    s = q @ k.T
    P = np.exp2(s - s.max(1, keepdims=True))
    return (P @ v) / P.sum(1, keepdims=True)


def _head(seed, R, N, gamma=None, recipe=False):
    """One head's fp16 q (scaled), k, v: LayerNorm-ed random vectors with a
    uniform gain `gamma` and no shift, or the synthetic workloads' affine
    recipe (gamma = 1 + N(0, 0.1), beta ~ N(0, 0.1) per feature)."""
    rng = np.random.default_rng(seed)
    if recipe:
        sd = math.sqrt(0.1)
        gq, bq = 1 + sd * rng.standard_normal(64), sd * rng.standard_normal(64)
        gk, bk = 1 + sd * rng.standard_normal(64), sd * rng.standard_normal(64)
    else:
        gq = gk = np.full(64, gamma)
        bq = bk = np.zeros(64)
    q = fp16(_ln(rng.standard_normal((R, 64)), gq, bq) * (LOG2E / 8))
    k = fp16(_ln(rng.standard_normal((N, 64)), gk, bk))
    v = fp16(rng.standard_normal((N, 64)))
    return q, k, v


def _row_rel(o, ref):
    return np.abs(o - ref).sum(1) / np.abs(ref).sum(1)


@pytest.mark.parametrize("gamma", [1.0, 1.9, 2.0, 2.05, 2.2])
def test_settle_rule_keeps_rows_precise_at_large_qk_gain(gamma):
    """A uniform QK-norm gain near 2 makes the logit bound loose enough that
    first-tile rows settle with a lifted reference; every row's attention
    output must still stay within fp16 round-off of the exact softmax (the
    online-max path measures <= 4.6e-4 per row here)."""
    q, k, v = _head(100 + int(gamma * 100), R=256, N=24744, gamma=gamma)
    o, _ = kernel_softmax_core(q, k, v)
    worst = _row_rel(o, _exact_core(q, k, v)).max()
    assert worst < 1e-3, (gamma, worst)


def test_wider_settle_gap_is_caught():
    """Planted mistake: the earlier gap of 29 (reference up to 14 above the row
    max) breaks the per-row bound at a gain of 2.05, so the check above has
    teeth."""
    q, k, v = _head(305, R=256, N=24744, gamma=2.05)
    o, _ = kernel_softmax_core(q, k, v, settle_gap=29.0)
    worst = _row_rel(o, _exact_core(q, k, v)).max()
    assert worst > 2e-3, worst


def test_synthetic_recipe_rows_settle_early():
    """With the workloads' QK-norm affine every row has settled after the
    eager tiles, so the measured kernel runs the cheap path (no per-tile row
    max) for the rest of the key loop."""
    q, k, v = _head(7, R=1024, N=24744, recipe=True)
    o, settled = kernel_softmax_core(q, k, v, tile=64)
    _, settled_early = kernel_softmax_core(q, k[:64 * EAGER_TILES], v[:64 * EAGER_TILES], tile=64)
    assert settled_early.all()
    assert _row_rel(o, _exact_core(q, k, v)).max() < 1e-3
