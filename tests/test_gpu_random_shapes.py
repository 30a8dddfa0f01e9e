"""GPU parity on seeded random shapes, at small sizes that the full oracle
finishes quickly.

The shapes vary the frames, both grid sides (zero included, i.e. special
tokens only), the width (d = 128, 256 or 1024) and the position offset. Each
shape runs every mode: frame, global, register, subsampled with random
windows, and a random query window of the global block. All are compared
element by element with the fp64 oracle at the block bar.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import avggt_sga
from vggt_global_attention_amd import api, configs, synth
from helpers import assert_parity, f64, oracle_params
from gpu_common import log, np64, require_gpu, run, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def shapes(n=10, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([128, 256, 1024], p=[0.45, 0.4, 0.15]))
        S = int(rng.integers(1, 7))
        gh, gw = int(rng.integers(0, 10)), int(rng.integers(0, 12))
        if gh == 0 or gw == 0:
            gh = gw = 0
        off = int(rng.integers(0, 3))
        sub = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        out.append((f"r{i}_S{S}_{gh}x{gw}_d{d}_o{off}", i, S, gh, gw, d, off, sub))
    return out


SHAPES = shapes()


@pytest.mark.parametrize("name,i,S,gh,gw,d,off,sub", SHAPES, ids=[s[0] for s in SHAPES])
def test_random_shape_all_modes(name, i, S, gh, gw, d, off, sub):
    w = configs.custom(name, S, gh, gw, d, d // 64, cid=400 + i)
    inp = synth.make_inputs(w)
    p = oracle_params(w, inp, pos_offset=off)
    d_in = to_dev(inp)
    X = f64(inp["X"])
    for mode, ref_fn in (("frame", oracle.frame_attention), ("global", oracle.global_attention),
                         ("register", oracle.register_attention)):
        log(f"[case] {name} {mode}")
        y = run(mode, w, d_in, pos_offset=off)
        assert_parity(np64(y), ref_fn(X, p), f"{name}/{mode}")
    if gh > 0:
        log(f"[case] {name} subsampled {sub}")
        y = run("subsampled", w, d_in, sub=sub, pos_offset=off)
        ref = avggt_sga.sga_attention(X, p, sub[0], sub[1])
        assert_parity(np64(y), ref, f"{name}/subsampled{sub}")
    rng = np.random.default_rng(len(name))
    begin = int(rng.integers(0, w.N))
    count = int(rng.integers(1, w.N - begin + 1))
    log(f"[case] {name} rows [{begin}, {begin + count})")
    blk = api.RowsBlock(d_in["X"], w.H, w.grid_h, w.grid_w, begin, count, pos_offset=off)
    y = blk(*[d_in[k] for k in ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")])
    rows = np.arange(begin, begin + count)
    ref = oracle.global_attention_rows(X, p, rows)
    assert_parity(np64(y), ref, f"{name}/rows")


@pytest.mark.parametrize("name,i,S,gh,gw,d,off,sub", SHAPES, ids=[s[0] for s in SHAPES])
def test_random_shape_bf16_operands_and_merged(name, i, S, gh, gw, d, off, sub):
    """The same shapes through the bf16-operand variant (its own bar) and
    the HTTM merged mode with random blocks and merge counts (per (token,
    head) against the oracle with Wo = I, near-tie pairs excluded)."""
    from oracle import httm as ohttm
    from helpers import BF16OPS_MAX, BF16OPS_MEAN, BF16OPS_RELL1, metrics
    import torch
    w = configs.custom(name, S, gh, gw, d, d // 64, cid=400 + i)
    inp = synth.make_inputs(w)
    p = oracle_params(w, inp, pos_offset=off)
    d_in = to_dev(inp)
    X = f64(inp["X"])
    for mode, ref_fn in (("frame", oracle.frame_attention), ("global", oracle.global_attention),
                         ("register", oracle.register_attention)):
        log(f"[case] {name} {mode} bf16 operands")
        m = metrics(np64(run(mode, w, d_in, pos_offset=off, operands="bf16")), ref_fn(X, p))
        assert m["nonfinite"] == 0 and m["relL1"] <= BF16OPS_RELL1, (name, mode, m)
        assert m["max_over_max"] <= BF16OPS_MAX and m["mean_over_max"] <= BF16OPS_MEAN, (name, m)
    rng = np.random.default_rng(7000 + i)
    F = int(rng.integers(2, 5))
    wh, ww = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    r = int(rng.integers(1, (F - 1) * wh * ww + 3))  # up to beyond a block's sources
    log(f"[case] {name} merged F={F} win={wh}x{ww} r={r}")
    inp_i = dict(inp)
    inp_i["Wo"] = torch.eye(d, dtype=inp["Wo"].dtype)
    d_i = to_dev(inp_i)
    p_i = oracle_params(w, inp_i, pos_offset=off)
    hp = ohttm.HttmParams(F, wh, ww, r)
    y = np64(run("merged", w, d_i, pos_offset=off, merge=(F, wh, ww, r))).reshape(w.N, w.H, -1)
    ref = ohttm.httm_attention(X, p_i, hp).reshape(w.N, w.H, -1)
    frag = ohttm.fragile(X, p_i, hp)
    assert np.isfinite(y).all()
    log(f"  {frag.sum()} of {frag.size} (token, head) pairs fragile")
    if (~frag).any():
        assert_parity(y[~frag], ref[~frag], f"{name}/merged")
