"""Pins for the fp64 oracle: brute force, closed forms, invariants, library cases.

Every check here ties the oracle to something other than itself: a pure-Python
re-derivation with complex-number rotations, a closed form the definition
implies, an invariant the pages fix, or a library routine (torch's LayerNorm,
scaled-dot-product attention and complex multiply) on a special case.  The
mutation tests at the end plant plausible mistakes in the oracle and check that
at least one pin catches each.
"""

from __future__ import annotations

import cmath
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import vggt_oracle as vo
from oracle import OracleParams
from vggt_global_attention_amd import configs, synth
from helpers import f64, oracle_params

RNG = np.random.default_rng(1234)


def small_case(S=2, gh=2, gw=3, d=32, H=2, seed=0, gscale=0.3, bscale=0.3):
    rng = np.random.default_rng(seed)
    T = 17 + gh * gw
    X = rng.standard_normal((S, T, d))
    p = OracleParams(
        Wqkv=rng.standard_normal((3 * d, d)) / math.sqrt(d),
        Wo=rng.standard_normal((d, d)) / math.sqrt(d),
        q_gamma=1 + gscale * rng.standard_normal((H, d // H)),
        q_beta=bscale * rng.standard_normal((H, d // H)),
        k_gamma=1 + gscale * rng.standard_normal((H, d // H)),
        k_beta=bscale * rng.standard_normal((H, d // H)),
        H=H, grid_h=gh, grid_w=gw)
    return X, p


# ----------------------------------------------------------------------------
# Brute force: pure Python, per token, RoPE as complex rotation
# ----------------------------------------------------------------------------

def _bf_token(x, p: OracleParams, t):
    d, H, Dh = p.d, p.H, p.Dh
    q4 = Dh // 4
    proj = [sum(p.Wqkv[o][i] * x[i] for i in range(d)) for o in range(3 * d)]
    heads = []
    for h in range(H):
        qkv = []
        for blk, (g, b) in enumerate(((p.q_gamma, p.q_beta), (p.k_gamma, p.k_beta), (None, None))):
            vec = proj[blk * d + h * Dh: blk * d + (h + 1) * Dh]
            if g is not None:
                mu = sum(vec) / Dh
                var = sum((z - mu) ** 2 for z in vec) / Dh
                vec = [(z - mu) / math.sqrt(var + p.ln_eps) * g[h][i] + b[h][i] for i, z in enumerate(vec)]
                if t >= 17:
                    pr = (t - 17) // p.grid_w + p.pos_offset
                    pc = (t - 17) % p.grid_w + p.pos_offset
                    out = list(vec)
                    for half, pos in ((0, pr), (1, pc)):
                        for i in range(q4):
                            lo = half * 2 * q4
                            z = complex(vec[lo + i], vec[lo + q4 + i])
                            z *= cmath.exp(1j * pos * p.rope_base ** (-i / q4))
                            out[lo + i], out[lo + q4 + i] = z.real, z.imag
                    vec = out
            qkv.append(vec)
        heads.append(qkv)
    return heads


def _bf_set(tokens, p: OracleParams):
    """tokens: list of (x, t_in_frame).  Returns list of output rows."""
    H, Dh, d = p.H, p.Dh, p.d
    feats = [_bf_token(x, p, t) for x, t in tokens]
    outs = []
    for a in range(len(tokens)):
        o = []
        for h in range(H):
            q = feats[a][h][0]
            logits = [sum(q[i] * feats[b][h][1][i] for i in range(Dh)) / math.sqrt(Dh)
                      for b in range(len(tokens))]
            m = max(logits)
            w = [math.exp(z - m) for z in logits]
            s = sum(w)
            o += [sum(w[b] * feats[b][h][2][i] for b in range(len(tokens))) / s for i in range(Dh)]
        outs.append([sum(p.Wo[j][i] * o[i] for i in range(d)) for j in range(d)])
    return outs


def test_bruteforce_global():
    X, p = small_case()
    S, T, d = X.shape
    toks = [(list(X[s, t]), t) for s in range(S) for t in range(T)]
    ref = np.array(_bf_set(toks, p)).reshape(S, T, d)
    got = oracle.global_attention(X, p, threads=1)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_bruteforce_frame():
    X, p = small_case(seed=1)
    S, T, d = X.shape
    ref = np.stack([np.array(_bf_set([(list(X[s, t]), t) for t in range(T)], p)) for s in range(S)])
    got = oracle.frame_attention(X, p, threads=1)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_bruteforce_register():
    X, p = small_case(S=3, seed=2)
    S, T, d = X.shape
    toks = [(list(X[s, t]), t) for s in range(S) for t in range(17)]
    spec = np.array(_bf_set(toks, p)).reshape(S, 17, d)
    got = oracle.register_attention(X, p, threads=1)
    assert np.abs(got[:, :17] - spec).max() <= 1e-12 * max(1.0, np.abs(spec).max())
    assert np.array_equal(got[:, 17:], X[:, 17:])


def test_bruteforce_pos_offset_and_base():
    X, p = small_case(seed=3)
    p.pos_offset = 1
    p.rope_base = 10000.0
    S, T, d = X.shape
    toks = [(list(X[s, t]), t) for s in range(S) for t in range(T)]
    ref = np.array(_bf_set(toks, p)).reshape(S, T, d)
    got = oracle.global_attention(X, p, threads=1)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


# ----------------------------------------------------------------------------
# Library special case: torch LayerNorm + complex RoPE + SDPA (fp64)
# ----------------------------------------------------------------------------

def _torch_block(X, p: OracleParams, mode: str):
    Xt = torch.from_numpy(X)
    S, T, d = X.shape
    H, Dh = p.H, p.Dh
    W = torch.from_numpy(p.Wqkv)
    q4 = Dh // 4

    def feats(rows, t):
        qkv = torch.nn.functional.linear(rows, W)
        q, k, v = qkv.split(d, dim=-1)
        q = q.reshape(-1, H, Dh)
        k = k.reshape(-1, H, Dh)
        v = v.reshape(-1, H, Dh)
        qn = torch.stack([torch.nn.functional.layer_norm(q[:, h], (Dh,), torch.from_numpy(p.q_gamma[h]),
                                                         torch.from_numpy(p.q_beta[h]), p.ln_eps) for h in range(H)], 1)
        kn = torch.stack([torch.nn.functional.layer_norm(k[:, h], (Dh,), torch.from_numpy(p.k_gamma[h]),
                                                         torch.from_numpy(p.k_beta[h]), p.ln_eps) for h in range(H)], 1)
        t = torch.as_tensor(t)
        patch = t >= 17
        pr = torch.where(patch, (t - 17) // p.grid_w, 0).double() + p.pos_offset
        pc = torch.where(patch, (t - 17) % p.grid_w, 0).double() + p.pos_offset
        inv = torch.tensor([p.rope_base ** (-i / q4) for i in range(q4)], dtype=torch.float64)

        def rot(x):
            out = x.clone()
            for half, pos in ((0, pr), (1, pc)):
                lo = half * 2 * q4
                z = torch.complex(x[..., lo:lo + q4], x[..., lo + q4:lo + 2 * q4])
                z = z * torch.polar(torch.ones_like(pos)[:, None], pos[:, None] * inv[None])[:, None, :]
                out[..., lo:lo + q4] = torch.where(patch[:, None, None], z.real, x[..., lo:lo + q4])
                out[..., lo + q4:lo + 2 * q4] = torch.where(patch[:, None, None], z.imag, x[..., lo + q4:lo + 2 * q4])
            return out
        return rot(qn), rot(kn), v

    def attend(rows, t):
        q, k, v = feats(rows, t)
        o = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1))
        o = o.transpose(0, 1).reshape(rows.shape[0], d)
        return torch.nn.functional.linear(o, torch.from_numpy(p.Wo))

    if mode == "global":
        return attend(Xt.reshape(S * T, d), torch.arange(T).repeat(S)).reshape(S, T, d).numpy()
    if mode == "frame":
        return torch.stack([attend(Xt[s], torch.arange(T)) for s in range(S)]).numpy()
    Y = Xt.clone()
    Y[:, :17] = attend(Xt[:, :17].reshape(S * 17, d), torch.arange(17).repeat(S)).reshape(S, 17, d)
    return Y.numpy()


@pytest.mark.parametrize("mode", ["global", "frame", "register"])
def test_library_case_torch(mode):
    X, p = small_case(S=3, gh=3, gw=4, d=64, H=4, seed=5)
    ref = _torch_block(X, p, mode)
    got = getattr(oracle, f"{mode}_attention")(X, p, threads=2)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_library_case_identity_rope_sdpa():
    """A 1x1 grid at position offset 0: the single patch sits at (0, 0), RoPE is
    the identity, and the block is textbook multi-head attention on LN'd q/k."""
    X, p = small_case(S=2, gh=1, gw=1, d=64, H=4, seed=6)
    Xt = torch.from_numpy(X).reshape(-1, 64)
    mha_q, mha_k, mha_v = torch.nn.functional.linear(Xt, torch.from_numpy(p.Wqkv)).split(64, -1)
    H, Dh = 4, 16
    qn = torch.nn.functional.layer_norm(mha_q.reshape(-1, H, Dh), (Dh,), eps=p.ln_eps) * torch.from_numpy(p.q_gamma) + torch.from_numpy(p.q_beta)
    kn = torch.nn.functional.layer_norm(mha_k.reshape(-1, H, Dh), (Dh,), eps=p.ln_eps) * torch.from_numpy(p.k_gamma) + torch.from_numpy(p.k_beta)
    o = torch.nn.functional.scaled_dot_product_attention(qn.transpose(0, 1), kn.transpose(0, 1),
                                                         mha_v.reshape(-1, H, Dh).transpose(0, 1))
    ref = torch.nn.functional.linear(o.transpose(0, 1).reshape(-1, 64), torch.from_numpy(p.Wo)).numpy()
    got = oracle.global_attention(X, p, threads=1).reshape(-1, 64)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------

def test_layernorm_closed_form():
    x = RNG.standard_normal((50, 3, 16)) * 2.5 + 0.7
    eps = 1e-5
    y = vo.layer_norm_heads(x, np.ones((3, 16)), np.zeros((3, 16)), eps)
    var = x.var(axis=-1)
    assert np.abs(y.mean(-1)).max() < 1e-14
    assert np.abs(y.var(-1) - var / (var + eps)).max() < 1e-13
    y2 = vo.layer_norm_heads(x, 2 * np.ones((3, 16)), 3 * np.ones((3, 16)), eps)
    assert np.abs(y2.mean(-1) - 3).max() < 1e-13
    assert np.abs(y2.var(-1) - 4 * var / (var + eps)).max() < 1e-12
    # per head: a head with a constant row gives beta exactly
    x[0, 1] = 5.0
    y3 = vo.layer_norm_heads(x, np.ones((3, 16)), np.full((3, 16), 0.25), eps)
    assert np.all(y3[0, 1] == 0.25)


def test_rope_unit_vectors():
    Dh, gw, base = 16, 7, 100.0
    q4 = Dh // 4
    r, c = 2, 5
    t = 17 + r * gw + c
    for i in range(q4):
        th = base ** (-i / q4)
        for half, pos in ((0, r), (1, c)):
            lo = half * 2 * q4
            e = np.zeros((1, 1, Dh))
            e[0, 0, lo + i] = 1.0
            y = vo.rope_2d(e, np.array([t]), gw, base)[0, 0]
            want = np.zeros(Dh)
            want[lo + i] = math.cos(pos * th)
            want[lo + q4 + i] = math.sin(pos * th)
            assert np.abs(y - want).max() < 1e-15
            e2 = np.zeros((1, 1, Dh))
            e2[0, 0, lo + q4 + i] = 1.0
            y2 = vo.rope_2d(e2, np.array([t]), gw, base)[0, 0]
            want2 = np.zeros(Dh)
            want2[lo + i] = -math.sin(pos * th)
            want2[lo + q4 + i] = math.cos(pos * th)
            assert np.abs(y2 - want2).max() < 1e-15
    # frequencies: theta_0 = 1 and a constant ratio base**(-1/q4) between neighbours
    ang = vo.rope_angles(np.array([1.0]), Dh, base)[0]
    assert ang[0] == 1.0
    assert np.allclose(ang[1:] / ang[:-1], base ** (-1 / q4), rtol=1e-14)
    # special tokens are not rotated
    x = RNG.standard_normal((17, 2, Dh))
    assert np.array_equal(vo.rope_2d(x, np.arange(17), gw, base), x)


def test_rope_relative_position_and_norm():
    Dh, gw = 64, 39
    q = RNG.standard_normal((1, 1, Dh))
    k = RNG.standard_normal((1, 1, Dh))
    ts = 17 + np.array([0, 5, 40, 200, 1013])
    for ta in ts:
        qa = vo.rope_2d(q, np.array([ta]), gw, 100.0)[0, 0]
        assert abs(np.linalg.norm(qa) - np.linalg.norm(q)) < 1e-13
    # <R(a) q, R(b) k> depends only on the grid displacement b - a
    pairs = [((0, 0), (1, 2)), ((3, 4), (4, 6)), ((10, 30), (11, 32))]
    vals = []
    for (ra, ca), (rb, cb) in pairs:
        qa = vo.rope_2d(q, np.array([17 + ra * gw + ca]), gw, 100.0)[0, 0]
        kb = vo.rope_2d(k, np.array([17 + rb * gw + cb]), gw, 100.0)[0, 0]
        vals.append(qa @ kb)
    assert max(vals) - min(vals) < 1e-12


def test_softmax_rows_sum_to_one():
    q = RNG.standard_normal((40, 16)) * 3
    k = RNG.standard_normal((70, 16)) * 3
    P = vo.attention_probs(q, k)
    assert np.abs(P.sum(1) - 1).max() < 1e-14
    assert (P > 0).all()
    # adding the same constant to every logit of a row leaves the row unchanged
    q2 = np.concatenate([q, np.full((40, 1), 2.0)], 1)
    k_one = np.concatenate([k, np.ones((70, 1))], 1)
    k_zero = np.concatenate([k, np.zeros((70, 1))], 1)
    assert np.abs(vo.attention_probs(q2, k_one) - vo.attention_probs(q2, k_zero)).max() < 1e-14


@pytest.mark.parametrize("mode", ["global", "frame", "register"])
def test_uniform_closed_form(mode):
    """Wq = 0 and beta_q = 0 make every logit zero: Y = mean over the set of V, times Wo^T."""
    X, p = small_case(S=3, gh=3, gw=4, d=64, H=4, seed=8)
    d = p.d
    p.Wqkv[:d] = 0.0
    p.q_beta[:] = 0.0
    got = getattr(oracle, f"{mode}_attention")(X, p, threads=2)
    V = X @ p.Wqkv[2 * d:].T
    if mode == "global":
        want = np.broadcast_to(V.reshape(-1, d).mean(0) @ p.Wo.T, got.shape)
        assert np.abs(got - want).max() < 1e-13
    elif mode == "frame":
        want = np.stack([np.broadcast_to(V[s].mean(0) @ p.Wo.T, got[s].shape) for s in range(X.shape[0])])
        assert np.abs(got - want).max() < 1e-13
    else:
        want = V[:, :17].reshape(-1, d).mean(0) @ p.Wo.T
        assert np.abs(got[:, :17] - want).max() < 1e-13
        assert np.array_equal(got[:, 17:], X[:, 17:])


@pytest.mark.parametrize("mode", ["global", "frame", "register"])
def test_identity_closed_form(mode):
    """Wk = Wq, gamma = 10, beta = 0: each token's own logit beats all others by
    hundreds, so attention is the identity and Y = V Wo^T."""
    X, p = small_case(S=3, gh=3, gw=4, d=64, H=4, seed=9)
    d = p.d
    p.Wqkv[d:2 * d] = p.Wqkv[:d]
    for a in (p.q_gamma, p.k_gamma):
        a[:] = 10.0
    for a in (p.q_beta, p.k_beta):
        a[:] = 0.0
    got = getattr(oracle, f"{mode}_attention")(X, p, threads=2)
    want = (X @ p.Wqkv[2 * d:].T) @ p.Wo.T
    if mode == "register":
        assert np.abs(got[:, :17] - want[:, :17]).max() < 1e-12
        assert np.array_equal(got[:, 17:], X[:, 17:])
    else:
        assert np.abs(got - want).max() < 1e-12


# ----------------------------------------------------------------------------
# Invariants fixed by the pages' definitions
# ----------------------------------------------------------------------------

def test_global_s1_equals_frame():
    X, p = small_case(S=1, seed=10)
    assert np.array_equal(oracle.global_attention(X, p, threads=1), oracle.frame_attention(X, p, threads=1))


def test_global_frame_permutation():
    """RoPE carries no frame index, so permuting frames permutes the output."""
    X, p = small_case(S=4, seed=11)
    perm = np.array([2, 0, 3, 1])
    a = oracle.global_attention(X, p, threads=1)
    b = oracle.global_attention(X[perm], p, threads=1)
    assert np.abs(a[perm] - b).max() < 1e-12 * np.abs(a).max()


def test_special_token_swap_across_frames():
    X, p = small_case(S=3, seed=12)
    Xs = X.copy()
    Xs[0, 3], Xs[2, 9] = X[2, 9].copy(), X[0, 3].copy()
    for fn in (oracle.global_attention, oracle.register_attention):
        a = fn(X, p, threads=1)
        b = fn(Xs, p, threads=1)
        assert np.abs(a[0, 3] - b[2, 9]).max() < 1e-12
        assert np.abs(a[2, 9] - b[0, 3]).max() < 1e-12


def test_frame_locality():
    X, p = small_case(S=3, seed=13)
    X2 = X.copy()
    X2[1] += 1.0
    a = oracle.frame_attention(X, p, threads=1)
    b = oracle.frame_attention(X2, p, threads=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    assert not np.allclose(a[1], b[1])


def test_register_semantics():
    X, p = small_case(S=3, seed=14)
    Y = oracle.register_attention(X, p, threads=1)
    assert np.array_equal(Y[:, 17:], X[:, 17:])
    # special outputs ignore patch tokens entirely
    X2 = X.copy()
    X2[:, 17:] = RNG.standard_normal(X2[:, 17:].shape)
    assert np.array_equal(oracle.register_attention(X2, p, threads=1)[:, :17], Y[:, :17])
    # one frame: register mode = frame attention over a patch-less frame
    p0 = OracleParams(**{**p.__dict__, "grid_h": 0, "grid_w": 1})
    X1 = X[:1, :17]
    assert np.abs(oracle.register_attention(X[:1], p, threads=1)[:, :17]
                  - oracle.frame_attention(X1, p0, threads=1)).max() < 1e-13


def test_frame_then_register_patch_rows():
    """Frame block followed by a register block: patch rows equal the frame output."""
    X, p = small_case(S=3, seed=15)
    F = oracle.frame_attention(X, p, threads=1)
    R = oracle.register_attention(F, p, threads=1)
    assert np.array_equal(R[:, 17:], F[:, 17:])


def test_linearity_power_of_two():
    X, p = small_case(S=2, seed=16)
    d = p.d
    Y = oracle.global_attention(X, p, threads=1)
    p2 = OracleParams(**{**p.__dict__, "Wo": p.Wo * 2})
    assert np.array_equal(oracle.global_attention(X, p2, threads=1), 2 * Y)
    W = p.Wqkv.copy()
    W[2 * d:] *= 2
    p3 = OracleParams(**{**p.__dict__, "Wqkv": W})
    assert np.array_equal(oracle.global_attention(X, p3, threads=1), 2 * Y)


@pytest.mark.parametrize("mode", ["global", "frame", "register"])
def test_rows_variants_match_full(mode):
    X, p = small_case(S=3, gh=3, gw=4, d=64, H=4, seed=17)
    S, T, d = X.shape
    full = getattr(oracle, f"{mode}_attention")(X, p, threads=2).reshape(S * T, d)
    rows = np.array([0, 5, 16, 17, 28, T, T + 20, 2 * T + 3, S * T - 1])
    got = getattr(oracle, f"{mode}_attention_rows")(X, p, rows, threads=2)
    assert np.abs(got - full[rows]).max() < 1e-12 * np.abs(full).max()


def test_synth_tiny_fp32_and_bf16():
    """The tiny workload: oracle runs on both the fp32 draws and their bf16 rounding."""
    w = configs.WORKLOADS["tiny"]
    i32 = synth.make_inputs(w, fp32=True)
    i16 = synth.make_inputs(w)
    assert i16["X"].dtype == torch.bfloat16 and i32["X"].dtype == torch.float32
    assert torch.equal(i16["X"], i32["X"].to(torch.bfloat16))
    for inp in (i32, i16):
        p = oracle_params(w, inp)
        Xg = f64(inp["X"])
        F = oracle.frame_attention(Xg, p)
        G = oracle.global_attention(F, p)
        assert np.isfinite(G).all() and G.shape == (w.S, w.T, w.d)


def test_synth_duplicates():
    w = configs.Workload("dup", 77, 12, 2, 3, 32, 2, ("global",), dup_frames=3)
    inp = synth.make_inputs(w)
    picks = inp["dup_frames"].tolist()
    assert len(picks) == 3 and picks == sorted(picks) and min(picks) >= 1
    for s in picks:
        diff = (inp["X"][s].float() - inp["X"][s - 1].float())
        assert diff.std().item() < 0.5


# ----------------------------------------------------------------------------
# Mutation checks: plausible mistakes planted in the oracle must trip a pin
# ----------------------------------------------------------------------------

def _library_pin_fails(monkeypatch, target, replacement):
    monkeypatch.setattr(vo, target, replacement)
    X, p = small_case(S=2, gh=2, gw=3, d=64, H=4, seed=21)
    ref = _torch_block(X, p, "global")
    got = oracle.global_attention(X, p, threads=1)
    return np.abs(got - ref).max() > 1e-9 * np.abs(ref).max()


def test_mutation_rope_frequency(monkeypatch):
    orig = vo.rope_2d

    def bad(x, t, gw, base, off=0):
        return orig(x, t, gw, 1.0 / base, off)
    assert _library_pin_fails(monkeypatch, "rope_2d", bad)


def test_mutation_rope_missing(monkeypatch):
    assert _library_pin_fails(monkeypatch, "rope_2d", lambda x, t, gw, base, off=0: x.copy())


def test_mutation_rope_direction(monkeypatch):
    orig = vo.rope_angles
    assert _library_pin_fails(monkeypatch, "rope_angles", lambda pos, dh, base: -orig(pos, dh, base))


def test_mutation_unbiased_variance(monkeypatch):
    def bad(x, g, b, eps):
        mu = x.mean(-1, keepdims=True)
        var = x.var(-1, ddof=1, keepdims=True)
        return (x - mu) / np.sqrt(var + eps) * g[None] + b[None]
    assert _library_pin_fails(monkeypatch, "layer_norm_heads", bad)


def test_mutation_softmax_scale(monkeypatch):
    def bad(qh, kh):
        a = qh @ kh.T / qh.shape[-1]
        e = np.exp(a - a.max(1, keepdims=True))
        return e / e.sum(1, keepdims=True)
    assert _library_pin_fails(monkeypatch, "attention_probs", bad)


def test_mutation_axis_swap(monkeypatch):
    orig = vo.token_positions

    def bad(t, gw):
        a, r, c = orig(t, gw)
        return a, c, r
    assert _library_pin_fails(monkeypatch, "token_positions", bad)
