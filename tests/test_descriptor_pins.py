"""Pins for the fp64 oracle of descriptor cross-attention (FlashVGGT reading).

Ties `oracle.descriptor` to: a pure-Python per-token construction, a torch
library case (layer_norm, complex-rotation RoPE, scaled_dot_product_attention,
linear), the global block it must reduce to when the descriptors are the
tokens themselves and nothing is rotated, a closed form for a single
descriptor, the chunk-recursive causality, and planted mistakes.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import descriptor as dsc
from oracle import vggt_oracle as vo
from test_oracle_pins import _bf_token, small_case


def _descs(M, d, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal((M, d))


def _bf_cross(X, D, p):
    """Pure Python: every token of X attends to the descriptors D."""
    S, T, d = X.shape
    H, Dh = p.H, p.Dh
    kv = [_bf_token(list(D[j]), p, 0) for j in range(len(D))]    # t = 0: not rotated
    out = []
    for s in range(S):
        for t in range(T):
            f = _bf_token(list(X[s, t]), p, t)
            o = []
            for h in range(H):
                q = f[h][0]
                lg = [sum(q[i] * kv[j][h][1][i] for i in range(Dh)) / math.sqrt(Dh)
                      for j in range(len(D))]
                m = max(lg)
                w = [math.exp(z - m) for z in lg]
                tot = sum(w)
                o += [sum(w[j] * kv[j][h][2][i] for j in range(len(D))) / tot for i in range(Dh)]
            out.append([sum(p.Wo[a][i] * o[i] for i in range(d)) for a in range(d)])
    return np.array(out).reshape(S, T, d)


def test_bruteforce_cross_attention():
    X, p = small_case(S=2, gh=2, gw=3, d=16, H=2, seed=21)
    D = _descs(7, 16, seed=22)
    got = dsc.descriptor_attention(X, D, p, threads=1)
    ref = _bf_cross(X, D, p)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _torch_cross(X, D, p):
    S, T, d = X.shape
    H, Dh = p.H, p.Dh
    q4 = Dh // 4
    W = torch.from_numpy(p.Wqkv)
    Xt = torch.from_numpy(X).reshape(S * T, d)
    Dt = torch.from_numpy(D)

    def ln(x, g, b):
        return torch.stack([torch.nn.functional.layer_norm(x[:, h], (Dh,), torch.from_numpy(g[h]),
                                                           torch.from_numpy(b[h]), p.ln_eps)
                            for h in range(H)], 1)

    q = ln(torch.nn.functional.linear(Xt, W[:d]).reshape(-1, H, Dh), p.q_gamma, p.q_beta)
    t = torch.arange(T).repeat(S)
    patch = t >= 17
    pr = torch.where(patch, (t - 17) // p.grid_w, 0).double() + p.pos_offset
    pc = torch.where(patch, (t - 17) % p.grid_w, 0).double() + p.pos_offset
    inv = torch.tensor([p.rope_base ** (-i / q4) for i in range(q4)], dtype=torch.float64)
    qr = q.clone()
    for half, pos in ((0, pr), (1, pc)):
        lo = half * 2 * q4
        z = torch.complex(q[..., lo:lo + q4], q[..., lo + q4:lo + 2 * q4])
        z = z * torch.polar(torch.ones_like(pos)[:, None], pos[:, None] * inv[None])[:, None, :]
        qr[..., lo:lo + q4] = torch.where(patch[:, None, None], z.real, q[..., lo:lo + q4])
        qr[..., lo + q4:lo + 2 * q4] = torch.where(patch[:, None, None], z.imag,
                                                   q[..., lo + q4:lo + 2 * q4])
    k = ln(torch.nn.functional.linear(Dt, W[d:2 * d]).reshape(-1, H, Dh), p.k_gamma, p.k_beta)
    v = torch.nn.functional.linear(Dt, W[2 * d:]).reshape(-1, H, Dh)
    o = torch.nn.functional.scaled_dot_product_attention(qr.transpose(0, 1), k.transpose(0, 1),
                                                         v.transpose(0, 1))
    o = o.transpose(0, 1).reshape(S * T, d)
    return torch.nn.functional.linear(o, torch.from_numpy(p.Wo)).reshape(S, T, d).numpy()


def test_library_case_torch():
    X, p = small_case(S=3, gh=3, gw=4, d=64, H=4, seed=23)
    D = _descs(19, 64, seed=24)
    got = dsc.descriptor_attention(X, D, p, threads=2)
    ref = _torch_cross(X, D, p)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_descriptors_equal_tokens_is_global_without_patches():
    # A grid without patches: every token is a camera / register token, so
    # nothing is rotated anywhere; with the tokens themselves as descriptors,
    # cross-attention is the global block.
    X, p = small_case(S=3, gh=0, gw=0, d=32, H=2, seed=25)
    got = dsc.descriptor_attention(X, X.reshape(-1, 32), p, threads=1)
    ref = vo.global_attention(X, p, threads=1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_single_descriptor_closed_form():
    # one key: its softmax weight is 1 for every query, Y = (D Wv^T) Wo^T
    X, p = small_case(S=2, gh=2, gw=2, d=32, H=2, seed=26)
    D = _descs(1, 32, seed=27)
    got = dsc.descriptor_attention(X, D, p, threads=1)
    ref = (D @ p.Wqkv[64:].T) @ p.Wo.T
    np.testing.assert_allclose(got, np.broadcast_to(ref, got.shape), rtol=0, atol=1e-12)


def test_descriptor_order_does_not_matter():
    X, p = small_case(S=2, gh=2, gw=3, d=32, H=2, seed=28)
    D = _descs(11, 32, seed=29)
    perm = np.random.default_rng(30).permutation(11)
    a = dsc.descriptor_attention(X, D, p, threads=1)
    b = dsc.descriptor_attention(X, D[perm], p, threads=1)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_rows_variant_matches_full():
    X, p = small_case(S=3, gh=2, gw=3, d=32, H=2, seed=31)
    D = _descs(9, 32, seed=32)
    full = dsc.descriptor_attention(X, D, p, threads=1).reshape(-1, 32)
    rows = np.array([0, 5, 16, 17, 22, 40, 68])
    np.testing.assert_allclose(dsc.descriptor_attention_rows(X, D, p, rows, threads=1),
                               full[rows], rtol=0, atol=1e-13)


def _chunk_pin(runner=None):
    """Chunk c's output is cross-attention to the descriptors of chunks 0..c
    and does not depend on later chunks."""
    runner = runner or dsc.chunk_recursive
    X, p = small_case(S=4, gh=2, gw=2, d=32, H=2, seed=33)
    Xc = [X[0:1], X[1:3], X[3:4]]
    Dc = [_descs(5, 32, 34), _descs(3, 32, 35), _descs(6, 32, 36)]
    out = runner(Xc, Dc, p, threads=1)
    for c in range(3):
        ref = dsc.descriptor_attention(Xc[c], np.concatenate(Dc[:c + 1]), p, threads=1)
        np.testing.assert_allclose(out[c], ref, rtol=0, atol=1e-13)
    Dc2 = Dc[:2] + [_descs(6, 32, 99)]
    out2 = runner(Xc, Dc2, p, threads=1)
    np.testing.assert_array_equal(out2[0], out[0])
    np.testing.assert_array_equal(out2[1], out[1])


def test_chunk_recursion_is_causal():
    _chunk_pin()


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _fails(fn, *a):
    try:
        fn(*a)
    except AssertionError:
        return True
    return False


def test_mutation_rotated_descriptors(monkeypatch):
    orig = vo._project

    def rotated(Xrows, t, p, want=("q", "k", "v")):
        if want == ("k", "v"):
            t = np.full_like(np.asarray(t), 17 + p.grid_w + 1)   # a patch position
        return orig(Xrows, t, p, want)
    monkeypatch.setattr(dsc, "_project", rotated)
    assert _fails(test_bruteforce_cross_attention)


def test_mutation_unnormalised_keys(monkeypatch):
    orig = vo._project

    def raw(Xrows, t, p, want=("q", "k", "v")):
        if want == ("k", "v"):
            out = orig(Xrows, t, p, ("v",))
            d, H, Dh = p.d, p.H, p.Dh
            out["k"] = (Xrows @ p.Wqkv[d:2 * d].T).reshape(-1, H, Dh)
            return out
        return orig(Xrows, t, p, want)
    monkeypatch.setattr(dsc, "_project", raw)
    assert _fails(test_library_case_torch)


def test_mutation_chunk_sees_only_its_own_descriptors():
    def own_only(Xc, Dc, p, threads=None):
        return [dsc.descriptor_attention(x, dd, p, threads) for x, dd in zip(Xc, Dc)]
    assert _fails(_chunk_pin, own_only)


def test_mutation_chunk_sees_future_descriptors():
    def all_of_them(Xc, Dc, p, threads=None):
        Dall = np.concatenate(Dc)
        return [dsc.descriptor_attention(x, Dall, p, threads) for x in Xc]
    assert _fails(_chunk_pin, all_of_them)

