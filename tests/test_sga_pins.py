"""Pins for the fp64 oracle of AVGGT subsampled global attention (SGA).

Each check ties `oracle.avggt_sga` to something other than itself: a
pure-Python construction of the mean-filled attention row, the global block
it must reduce to, a library softmax attention on a case where mean filling is
exact, closed forms, and planted mistakes that the pins must catch.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import avggt_sga as sg
from oracle import vggt_oracle as vo
from test_oracle_pins import small_case


def _rand_qkv(N=37, H=2, Dh=8, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    q = scale * rng.standard_normal((N, H, Dh))
    k = scale * rng.standard_normal((N, H, Dh))
    v = rng.standard_normal((N, H, Dh))
    return q, k, v


def _bf_filled_row(q, k, v, kept, i, h):
    """Pure Python: row i of the full N-column attention in which every column
    that is neither kept nor i itself holds the mean of the discarded keys and
    values."""
    N, Dh = len(k), len(k[0][0])
    D = [j for j in range(N) if not kept[j]]
    kbar = [sum(k[j][h][e] for j in D) / len(D) for e in range(Dh)] if D else None
    vbar = [sum(v[j][h][e] for j in D) / len(D) for e in range(Dh)] if D else None
    logits, vals = [], []
    for j in range(N):
        if kept[j] or j == i:
            kj, vj = k[j][h], v[j][h]
        else:
            kj, vj = kbar, vbar
        logits.append(sum(q[i][h][e] * kj[e] for e in range(Dh)) / math.sqrt(Dh))
        vals.append(vj)
    m = max(logits)
    w = [math.exp(a - m) for a in logits]
    tot = sum(w)
    return [sum(w[j] * vals[j][e] for j in range(N)) / tot for e in range(Dh)]


def _kept_mask(N, seed, frac=0.35):
    rng = np.random.default_rng(seed)
    kept = rng.random(N) < frac
    kept[0] = True
    return kept


def test_kept_tokens_closed_form():
    for S, gh, gw, sh, sw in ((2, 8, 8, 3, 3), (3, 26, 39, 3, 3), (1, 5, 7, 2, 4), (2, 4, 4, 1, 1),
                              (1, 3, 3, 5, 5), (2, 0, 0, 2, 2)):
        kept = sg.kept_tokens(S, gh, gw, sh, sw)
        T = 17 + gh * gw
        assert kept.shape == (S * T,)
        per = 17 + (-(-gh // sh)) * (-(-gw // sw)) if gh * gw else 17
        assert kept.sum() == S * per
        for s in range(S):
            assert kept[s * T:s * T + 17].all()           # specials always kept
            for r in range(gh):
                for c in range(gw):
                    assert kept[s * T + 17 + r * gw + c] == (r % sh == 0 and c % sw == 0)


def test_sga_bruteforce_filled_rows():
    q, k, v = _rand_qkv(N=29, H=2, Dh=8, seed=3)
    kept = _kept_mask(29, seed=4)
    rows = np.arange(29)
    O = sg.sga_core(q, k, v, kept, threads=1).reshape(29, 2, 8)
    for i in rows:
        for h in range(2):
            ref = _bf_filled_row(q.tolist(), k.tolist(), v.tolist(), kept.tolist(), int(i), h)
            np.testing.assert_allclose(O[i, h], ref, rtol=0, atol=1e-12)


def test_sga_rows_subset_matches_all_rows():
    q, k, v = _rand_qkv(N=64, H=3, Dh=8, seed=5)
    kept = _kept_mask(64, seed=6)
    full = sg.sga_core(q, k, v, kept, threads=2)
    rows = np.array([0, 5, 17, 40, 63])
    part = sg.sga_core(q[rows], k, v, kept, rows=rows, threads=1, chunk=2)
    np.testing.assert_allclose(part, full[rows], rtol=0, atol=1e-13)


def test_sga_no_subsampling_is_global():
    X, p = small_case(S=2, gh=3, gw=4, d=32, H=2, seed=11)
    y = sg.sga_attention(X, p, 1, 1, threads=1)
    ref = vo.global_attention(X, p, threads=1)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def _torch_full_attention(q, k, v):
    qt = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2)
    kt = torch.tensor(k, dtype=torch.float64).permute(1, 0, 2)
    vt = torch.tensor(v, dtype=torch.float64).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o.permute(1, 0, 2).reshape(q.shape[0], -1).numpy()


def _equal_discarded_case(seed=7):
    q, k, v = _rand_qkv(N=48, H=2, Dh=8, seed=seed)
    kept = _kept_mask(48, seed=seed + 1, frac=0.3)
    D = ~kept
    k[D] = k[np.nonzero(D)[0][0]]     # every discarded key equal ...
    v[D] = v[np.nonzero(D)[0][1]]     # ... and every discarded value
    return q, k, v, kept


def test_sga_exact_when_discarded_columns_are_equal():
    # Mean filling replaces each discarded column by the mean pair; if all
    # discarded keys and values are equal, that is no approximation at all.
    q, k, v, kept = _equal_discarded_case()
    y = sg.sga_core(q, k, v, kept, threads=1)
    np.testing.assert_allclose(y, _torch_full_attention(q, k, v), rtol=0, atol=1e-12)


def test_sga_uniform_closed_form():
    # q = 0: every column of the filled row weighs 1/N.
    q, k, v = _rand_qkv(N=40, H=2, Dh=8, seed=9)
    q[:] = 0.0
    kept = _kept_mask(40, seed=10)
    D = np.nonzero(~kept)[0]
    vbar = v[D].mean(axis=0)
    vk = v[kept].sum(axis=0)
    O = sg.sga_core(q, k, v, kept, threads=1).reshape(40, 2, 8)
    for i in range(40):
        if kept[i]:
            ref = (vk + len(D) * vbar) / 40
        else:
            ref = (vk + v[i] + (len(D) - 1) * vbar) / 40
        np.testing.assert_allclose(O[i], ref, rtol=0, atol=1e-13)


def test_sga_rows_variant_matches_full_block():
    X, p = small_case(S=3, gh=4, gw=5, d=32, H=2, seed=12)
    full = sg.sga_attention(X, p, 2, 3, threads=1).reshape(-1, 32)
    rows = np.array([0, 16, 17, 18, 37, 80, 110])
    part = sg.sga_attention_rows(X, p, 2, 3, rows, threads=1)
    np.testing.assert_allclose(part, full[rows], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin above fail
# ----------------------------------------------------------------------------

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_mutation_mean_counted_once(monkeypatch):
    monkeypatch.setattr(sg, "mean_multiplicity", lambda nD, diag_on: np.minimum(1, nD - diag_on))
    assert _fails(test_sga_exact_when_discarded_columns_are_equal)
    assert _fails(test_sga_bruteforce_filled_rows)


def test_mutation_diagonal_dropped(monkeypatch):
    monkeypatch.setattr(sg, "diagonal_columns", lambda kept_rows: np.zeros_like(kept_rows))
    assert _fails(test_sga_bruteforce_filled_rows)
    assert _fails(test_sga_uniform_closed_form)


def test_mutation_window_anchor(monkeypatch):
    # keeping the last cell of each window instead of the first
    def shifted(S, gh, gw, sh, sw):
        T = 17 + gh * gw
        t = np.arange(T)
        pidx = t - 17
        r, c = pidx // max(gw, 1), pidx % max(gw, 1)
        return np.tile((t < 17) | ((r % sh == sh - 1) & (c % sw == sw - 1)), S)
    monkeypatch.setattr(sg, "kept_tokens", shifted)
    assert _fails(test_kept_tokens_closed_form)
