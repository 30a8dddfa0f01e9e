"""Pins of the HTTM merging oracle (oracle/httm.py) -- CPU only.

"HTTM: Head-wise Temporal Token Merging for Faster VGGT" (10100.com) gives
the method's parts (section 02: head-wise merging, block-wise matching,
temporal reordering into spatio-temporal blocks) but no formula, so the
oracle's reading is pinned by:
* a pure-Python per-token construction of the same reading (blocks,
  similarities, best destinations, the r best sources, means, size-weighted
  softmax, unmerging), written without the oracle's vectorised code;
* the similarity emulation (fp16 keys, fp32 sums in feature order) against
  NumPy's own float32 arithmetic;
* r = 0: exactly the global block;
* exact duplicates: with every frame run made of identical frames, a uniform
  QK-norm gain and no shift, every source's best destination is its own twin
  (Cauchy-Schwarz on equal-norm keys) and merging all sources reproduces the
  global block exactly -- a merged token of size n stands for n identical
  keys and values;
* the uniform closed form: with zero queries every logit is 0 and the output
  is the mean value over all tokens whatever merges (the size weights make
  the merged sum equal the token sum);
* the merged length N - sum_b min(r, sources_b), the same in every head;
* planted mistakes -- no size weight, summed instead of averaged values,
  one head's decisions for all heads, the run's last frame as destinations,
  a ranking that prefers the lowest similarity -- each fail one of the above.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import httm
from test_oracle_pins import _bf_token, small_case


def bf_httm(X, p, hp):
    """Pure-Python reading of the method, token by token."""
    S, T, d = X.shape
    H, Dh = p.H, p.Dh
    gh, gw = p.grid_h, p.grid_w
    feats = {(s, t): _bf_token(list(X[s, t]), p, t) for s in range(S) for t in range(T)}
    # blocks: frame runs x windows, destinations = the run's first frame
    blocks = []
    for f0 in range(0, S, hp.frames):
        run = list(range(f0, min(S, f0 + hp.frames)))
        for r0 in range(0, gh, hp.win_h):
            for c0 in range(0, gw, hp.win_w):
                cells = [17 + r * gw + c for r in range(r0, min(gh, r0 + hp.win_h))
                         for c in range(c0, min(gw, c0 + hp.win_w))]
                blocks.append(([(run[0], t) for t in cells],
                               [(s, t) for s in run[1:] for t in cells]))
    out = {}
    for h in range(H):
        # decisions in the kernels' precision: fp16 keys, fp32 sums in feature order
        key = lambda tok: [float(np.float16(x)) for x in feats[tok][h][1]]  # noqa: E731

        def sim32(ka, kb):
            acc = np.float32(0.0)
            for x, y in zip(ka, kb):
                acc = np.float32(acc + np.float32(x) * np.float32(y))
            return float(acc)
        groups = [[(s, t)] for s in range(S) for t in range(17)]
        for dst, src in blocks:
            best, score = [], []
            for a in src:
                sims = [sim32(key(a), key(b)) for b in dst]
                j = max(range(len(dst)), key=lambda i: (sims[i], -i))
                best.append(j)
                score.append(sims[j])
            ranked = sorted(range(len(src)), key=lambda i: (-score[i], i))
            merged = set(ranked[:min(hp.r, len(src))])
            for j, b in enumerate(dst):
                groups.append([b] + [src[i] for i in range(len(src)) if i in merged and best[i] == j])
            groups += [[src[i]] for i in range(len(src)) if i not in merged]
        mean = [[[sum(feats[m][h][c][i] for m in g) / len(g) for i in range(Dh)] for g in groups]
                for c in range(3)]
        for gi, g in enumerate(groups):
            q = mean[0][gi]
            logits = [sum(x * y for x, y in zip(q, mean[1][gj])) / math.sqrt(Dh)
                      + math.log(len(groups[gj])) for gj in range(len(groups))]
            mx = max(logits)
            w = [math.exp(z - mx) for z in logits]
            o = [sum(w[gj] * mean[2][gj][i] for gj in range(len(groups))) / sum(w)
                 for i in range(Dh)]
            for tok in g:
                out.setdefault(tok, [None] * H)[h] = o
    Y = np.empty((S, T, d))
    for (s, t), heads in out.items():
        o = [z for hh in heads for z in hh]
        Y[s, t] = [sum(p.Wo[j][i] * o[i] for i in range(d)) for j in range(d)]
    return Y


def test_similarities_are_fp32_sums_of_fp16_products():
    rng = np.random.default_rng(12)
    a = rng.standard_normal((3, 5, 64)) * 3
    b = rng.standard_normal((3, 4, 64)) * 3
    got = httm.similarities(a, b)
    a16, b16 = a.astype(np.float16).astype(np.float32), b.astype(np.float16).astype(np.float32)
    for i in range(3):
        for s_ in range(5):
            for d_ in range(4):
                acc = np.float32(0.0)
                for f in range(64):
                    acc = np.float32(acc + a16[i, s_, f] * b16[i, d_, f])
                assert got[i, s_, d_] == float(acc)
    # and not the fp64 dot of the unrounded keys
    assert not np.array_equal(got, np.einsum("bsf,bdf->bsd", a, b))


def close(a, b, tol=1e-12):
    return np.abs(a - b).max() <= tol * max(1.0, np.abs(b).max())


@pytest.mark.parametrize("S,gh,gw,hp", [
    (4, 2, 3, httm.HttmParams(2, 1, 2, 2)),    # whole windows, F = 2
    (5, 3, 4, httm.HttmParams(3, 2, 3, 4)),    # ragged windows, a short last run
    (3, 2, 3, httm.HttmParams(2, 2, 3, 99)),   # r above the sources: all merge
])
def test_bruteforce(S, gh, gw, hp):
    X, p = small_case(S=S, gh=gh, gw=gw, d=32, H=2, seed=S + gh)
    assert close(httm.httm_attention(X, p, hp), bf_httm(X, p, hp))


def test_no_merge_is_global():
    X, p = small_case(S=4, gh=4, gw=6, d=64, H=2, seed=5)
    assert close(httm.httm_attention(X, p, httm.HttmParams(2, 2, 3, 0)),
                 oracle.global_attention(X, p, threads=1))


def duplicate_case(F=2, S=4, gh=4, gw=6):
    """Frames of each run identical; uniform QK-norm gain, no shift."""
    X, p = small_case(S=S, gh=gh, gw=gw, d=64, H=2, seed=7)
    for f0 in range(0, S, F):
        X[f0:f0 + F] = X[f0]
    for a in (p.q_gamma, p.k_gamma):
        a[:] = 1.3
    for a in (p.q_beta, p.k_beta):
        a[:] = 0.0
    return X, p


@pytest.mark.parametrize("F", [2, 3])
def test_duplicate_frames_merge_into_twins_and_match_global(F):
    X, p = duplicate_case(F=F, S=6)
    hp = httm.HttmParams(F, 2, 3, 99)
    S, T, _ = X.shape
    k = httm._qkv(X, p, want=("k",))["k"]
    for h in range(p.H):
        owner, n = httm.head_owner(k[:, h], S, p.grid_h, p.grid_w, hp)
        t = np.arange(S * T)
        patch = (t % T) >= 17
        twin = (t // T // F * F) * T + t % T
        assert np.array_equal(owner[patch], owner[twin[patch]])
        assert set(np.unique(n)) <= {1.0, float(F)}
    assert close(httm.httm_attention(X, p, hp), oracle.global_attention(X, p, threads=1), 1e-10)


def test_uniform_closed_form():
    X, p = small_case(S=4, gh=4, gw=6, d=64, H=2, seed=8)
    p.Wqkv[:p.d] = 0
    p.q_beta[:] = 0
    hp = httm.HttmParams(2, 2, 3, 4)
    S, T, d = X.shape
    Xf = X.reshape(-1, d)
    ref = (Xf.mean(0) @ p.Wqkv[2 * d:].T) @ p.Wo.T
    y = httm.httm_attention(X, p, hp).reshape(-1, d)
    assert close(y, np.broadcast_to(ref, y.shape))


def test_merged_length_same_in_every_head():
    X, p = small_case(S=5, gh=3, gw=4, d=64, H=2, seed=9)
    hp = httm.HttmParams(2, 2, 3, 3)
    S, T, _ = X.shape
    k = httm._qkv(X, p, want=("k",))["k"]
    M = httm.merged_length(S, p.grid_h, p.grid_w, hp)
    expect = S * T - sum(min(hp.r, len(src)) for _, src in httm.blocks(S, p.grid_h, p.grid_w, hp))
    assert M == expect < S * T
    owners = []
    for h in range(p.H):
        owner, n = httm.head_owner(k[:, h], S, p.grid_h, p.grid_w, hp)
        assert len(n) == M and n.sum() == S * T and n.min() >= 1
        owners.append(owner)
    assert not np.array_equal(owners[0], owners[1])  # the heads decide differently here


def test_rows_variant_matches_full():
    X, p = small_case(S=5, gh=3, gw=4, d=64, H=2, seed=10)
    hp = httm.HttmParams(2, 2, 2, 2)
    y = httm.httm_attention(X, p, hp).reshape(-1, p.d)
    rows = np.array([0, 16, 17, 30, 58, 95, 140, 144])
    assert close(httm.httm_attention_rows(X, p, hp, rows), y[rows])


def test_fragile_flags_a_near_tie():
    """Copying one destination's token state onto its neighbour cell gives two
    destinations whose keys differ only by a one-cell rotation: the sources'
    best destination is then decided by a hair, and the block's tokens are
    flagged in more heads than before."""
    X, p = small_case(S=2, gh=1, gw=4, d=64, H=2, seed=11)
    hp = httm.HttmParams(2, 1, 2, 1)
    T = X.shape[1]
    frag0 = httm.fragile(X, p, hp)
    X[0, 18] = X[0, 17]
    frag = httm.fragile(X, p, hp)
    assert frag.shape == (2 * T, 2)
    assert frag0.sum() < frag.sum()
    assert not frag[:17].any() and not frag[T:T + 17].any()   # special tokens never merge


def test_fragile_rows_form_matches_full():
    X, p = small_case(S=5, gh=3, gw=7, d=128, H=2, seed=12)
    hp = httm.HttmParams(3, 2, 3, 4)
    full = httm.fragile(X, p, hp)
    rows = np.array([0, 17, 30, 40, 2 * X.shape[1] + 20, 4 * X.shape[1] + 37])
    assert np.array_equal(httm.fragile(X, p, hp, rows=rows), full[rows])


# ----------------------------------------------------------------------------
# Planted mistakes: each must break a pin above
# ----------------------------------------------------------------------------

def _merged_attention_variant(weighted=True, summed_values=False):
    """merged_attention with one step changed (for the planted mistakes)."""
    def fn(q, k, v, owner, n, query_groups=None):
        acc = [np.zeros((len(n), q.shape[1])) for _ in range(3)]
        for a, x in zip(acc, (q, k, v)):
            np.add.at(a, owner, x)
        qm, km = acc[0] / n[:, None], acc[1] / n[:, None]
        vm = acc[2] if summed_values else acc[2] / n[:, None]
        if query_groups is not None:
            qm = qm[query_groups]
        a = qm @ km.T / math.sqrt(q.shape[1])
        if weighted:
            a = a + np.log(n)[None, :]
        w = np.exp(a - a.max(axis=1, keepdims=True))
        return (w @ vm) / w.sum(axis=1, keepdims=True)
    return fn


def test_mistake_no_size_weight(monkeypatch):
    monkeypatch.setattr(httm, "merged_attention", _merged_attention_variant(weighted=False))
    X, p = duplicate_case()
    got = httm.httm_attention(X, p, httm.HttmParams(2, 2, 3, 99))
    assert not close(got, oracle.global_attention(X, p, threads=1), 1e-6)


def test_mistake_summed_values(monkeypatch):
    monkeypatch.setattr(httm, "merged_attention", _merged_attention_variant(summed_values=True))
    X, p = small_case(S=4, gh=4, gw=6, d=64, H=2, seed=8)
    p.Wqkv[:p.d] = 0
    p.q_beta[:] = 0
    d = p.d
    ref = (X.reshape(-1, d).mean(0) @ p.Wqkv[2 * d:].T) @ p.Wo.T
    y = httm.httm_attention(X, p, httm.HttmParams(2, 2, 3, 4)).reshape(-1, d)
    assert not close(y, np.broadcast_to(ref, y.shape), 1e-6)


def test_mistake_one_head_decides(monkeypatch):
    real = httm.head_owner
    first = {}

    def shared(kh, S, gh, gw, hp):
        if "o" not in first:
            first["o"] = real(kh, S, gh, gw, hp)
        return first["o"]
    monkeypatch.setattr(httm, "head_owner", shared)
    S, gh, gw = 5, 3, 4
    hp = httm.HttmParams(3, 2, 3, 4)
    X, p = small_case(S=S, gh=gh, gw=gw, d=32, H=2, seed=S + gh)
    assert not close(httm.httm_attention(X, p, hp), bf_httm(X, p, hp), 1e-6)


def test_mistake_last_frame_destinations(monkeypatch):
    real = httm.blocks

    def last(S, gh, gw, hp):
        out = []
        for dst, src in real(S, gh, gw, hp):
            if len(src):
                allt = np.concatenate((dst, src)).reshape(-1, len(dst))
                dst, src = allt[-1], allt[:-1].ravel()
            out.append((dst, src))
        return out
    monkeypatch.setattr(httm, "blocks", last)
    S, gh, gw = 4, 2, 3
    hp = httm.HttmParams(2, 1, 2, 2)
    X, p = small_case(S=S, gh=gh, gw=gw, d=32, H=2, seed=S + gh)
    monkeypatch.setattr(httm, "blocks", real)
    ref = bf_httm(X, p, hp)
    monkeypatch.setattr(httm, "blocks", last)
    assert not close(httm.httm_attention(X, p, hp), ref, 1e-6)


def test_mistake_lowest_similarity_first(monkeypatch):
    def lowest(kh, dst, src, r):
        B, ns = src.shape
        sim = np.einsum("bsf,bdf->bsd", kh[src], kh[dst])
        best = np.argmax(sim, axis=2)
        score = np.take_along_axis(sim, best[..., None], axis=2)[..., 0]
        order = np.argsort(score, axis=1, kind="stable")   # ascending: the mistake
        merged = np.zeros((B, ns), dtype=bool)
        np.put_along_axis(merged, order[:, :min(r, ns)], True, axis=1)
        return best, merged
    S, gh, gw = 5, 3, 4
    hp = httm.HttmParams(3, 2, 3, 4)
    X, p = small_case(S=S, gh=gh, gw=gw, d=32, H=2, seed=S + gh)
    ref = bf_httm(X, p, hp)
    monkeypatch.setattr(httm, "block_decisions", lowest)
    assert not close(httm.httm_attention(X, p, hp), ref, 1e-6)
