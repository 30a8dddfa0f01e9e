"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar (the parity tolerance for bf16 inputs / fp32 accumulation):
max|err| <= 1e-2 * max|ref| and relL1 = sum|err| / sum|ref| <= 2e-3 ("mean
relative error" read as the L1 ratio, which stays defined where ref is near 0).  Sizes: the tiny
alternating block and ragged shapes with the full oracle, the 24-frame layer
with the full oracle, and the 100/300/500-frame layers on seeded row samples
plus closed forms that hold at full size.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from vggt_global_attention_amd import api, configs, synth
from vggt_global_attention_amd import binding as B
from helpers import assert_parity, f64, oracle_params
from gpu_common import log, np64, require_gpu, run, to_dev

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
ORACLE = {"frame": oracle.frame_attention, "global": oracle.global_attention,
          "register": oracle.register_attention}
ORACLE_ROWS = {"frame": oracle.frame_attention_rows, "global": oracle.global_attention_rows,
               "register": oracle.register_attention_rows}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def full_case(w, mode, inp=None, label=None):
    inp = inp or synth.make_inputs(w)
    log(f"[case] {label or w.name} mode={mode} S={w.S} T={w.T} d={w.d} H={w.H}")
    d = to_dev(inp)
    y = run(mode, w, d)
    ref = ORACLE[mode](f64(inp["X"]), oracle_params(w, inp))
    return assert_parity(np64(y), ref, f"{w.name}/{mode}")


@pytest.mark.parametrize("mode", ["frame", "global", "register"])
def test_tiny(mode):
    full_case(W["tiny"], mode)


def test_tiny_alternating_block():
    """The tiny alternating block: frame attention, then global attention on its output."""
    w = W["tiny"]
    inp = synth.make_inputs(w)
    p = oracle_params(w, inp)
    d = to_dev(inp)
    f_gpu = run("frame", w, d)
    g_gpu = run("global", w, d, X=f_gpu)
    f_ref = oracle.frame_attention(f64(inp["X"]), p)
    f_ref16 = torch.from_numpy(f_ref).to(torch.bfloat16)
    g_ref = oracle.global_attention(f64(f_ref16), p)
    assert_parity(np64(f_gpu), f_ref, "tiny/frame")
    assert_parity(np64(g_gpu), g_ref, "tiny/frame->global")


RAGGED = [
    configs.custom("ragged", 3, 5, 7, 128, 2, cid=11),     # T = 52: one partial key tile
    configs.custom("ragged2", 2, 7, 11, 256, 4, cid=12),   # T = 94: tile + 30-key tail
    configs.custom("patchless", 1, 0, 0, 128, 2, cid=13),  # T = 17: specials only
    configs.custom("onerow", 5, 1, 1, 128, 2, cid=14),     # T = 18: 1x1 grid
    configs.custom("wide", 4, 9, 30, 128, 2, cid=15),      # T = 287, N = 1148
    # last key tile of a frame at the edges of the short-tile path (at most 32
    # valid keys: only the tile's first half runs)
    configs.custom("edge32", 2, 1, 79, 128, 2, cid=16),    # T = 96: 32-key tail (short path)
    configs.custom("edge33", 2, 8, 10, 128, 2, cid=17),    # T = 97: 33-key tail (whole tile)
    configs.custom("edge64", 2, 1, 47, 128, 2, cid=18),    # T = 64: no tail
    configs.custom("edge65", 2, 6, 8, 128, 2, cid=19),     # T = 65: 1-key tail
]


@pytest.mark.parametrize("w", RAGGED, ids=[r.name for r in RAGGED])
@pytest.mark.parametrize("mode", ["frame", "global", "register"])
def test_ragged_shapes(w, mode):
    full_case(w, mode)


@pytest.mark.parametrize("mode", ["global", "frame"])
def test_s24_full_oracle(mode):
    full_case(W["s24"], mode)


def sampled_case(w, mode, n_rows=384, inp=None):
    inp = inp or synth.make_inputs(w)
    log(f"[case] {w.name} mode={mode} sampled rows={n_rows}")
    d = to_dev(inp)
    y = run(mode, w, d)
    rows = synth.sample_rows(w, n_rows).numpy()
    got = np64(y).reshape(-1, w.d)[rows]
    ref = ORACLE_ROWS[mode](f64(inp["X"]), oracle_params(w, inp), rows)
    return assert_parity(got, ref, f"{w.name}/{mode}/sampled")


def test_s100_global_sampled():
    sampled_case(W["s100"], "global")


def test_s300_global_sampled():
    sampled_case(W["s300"], "global", n_rows=256)


def test_s500_global_sampled():
    """The largest global set of the workloads: 500 frames, 515,500 tokens
    (q/k/v offsets past 2^31 bytes, 8,055 key tiles, a split tail)."""
    sampled_case(W["s500"], "global", n_rows=128)


def test_s500_frame_sampled():
    sampled_case(W["s500"], "frame")


def test_s500_register_full():
    """Register mode at 500 frames: 8,500 special tokens, full oracle."""
    full_case(W["s500"], "register")


# ----------------------------------------------------------------------------
# Closed forms at full size (no oracle run over N^2)
# ----------------------------------------------------------------------------

def uniform_inputs(w):
    inp = synth.make_inputs(w)
    inp["Wqkv"] = inp["Wqkv"].clone()
    inp["Wqkv"][: w.d] = 0
    inp["q_beta"] = torch.zeros_like(inp["q_beta"])
    return inp


@pytest.mark.parametrize("name", ["s100", "s300"])
def test_uniform_closed_form_full(name):
    """Wq = 0, beta_q = 0: every logit is 0, so Y = mean over all tokens of v, times Wo^T."""
    w = W[name]
    inp = uniform_inputs(w)
    log(f"[case] {name} uniform closed form")
    y = np64(run("global", w, to_dev(inp))).reshape(-1, w.d)
    X = f64(inp["X"]).reshape(-1, w.d)
    Wv = f64(inp["Wqkv"])[2 * w.d:]
    vmean = (X.sum(0) / X.shape[0]) @ Wv.T
    ref = np.broadcast_to(vmean @ f64(inp["Wo"]).T, y.shape)
    assert_parity(y, ref, f"{name}/uniform")


def identity_inputs(w):
    inp = synth.make_inputs(w)
    W_ = inp["Wqkv"].clone()
    W_[w.d: 2 * w.d] = W_[: w.d]
    inp["Wqkv"] = W_
    for k in ("q_gamma", "k_gamma"):
        inp[k] = torch.full_like(inp[k], 10.0)
    for k in ("q_beta", "k_beta"):
        inp[k] = torch.zeros_like(inp[k])
    return inp


@pytest.mark.parametrize("name,mode", [("s100", "global"), ("s24", "frame"), ("s500", "register")])
def test_identity_closed_form(name, mode):
    """Wk = Wq, gamma = 10, beta = 0: each token's own logit wins by hundreds,
    so attention is the identity and Y = (x Wv^T) Wo^T on every row."""
    w = W[name]
    inp = identity_inputs(w)
    log(f"[case] {name} identity closed form ({mode})")
    y = np64(run(mode, w, to_dev(inp))).reshape(-1, w.d)
    rows = synth.sample_rows(w, 512).numpy()
    if mode == "register":
        rows = np.array([r for r in range(w.N) if r % w.T < 17][::7])
    X = f64(inp["X"]).reshape(-1, w.d)[rows]
    ref = (X @ f64(inp["Wqkv"])[2 * w.d:].T) @ f64(inp["Wo"]).T
    assert_parity(y[rows], ref, f"{name}/identity")


# ----------------------------------------------------------------------------
# Large QK-norm gain: the softmax reference rule under a loose logit bound
# ----------------------------------------------------------------------------
# With a uniform QK-norm gain near 2 (beta = 0) the bound |q| max|k| sits far
# above a row's first-tile max, the band where a pinned reference could float
# above the row's true max.  Per-row bar: the fp16-inside design itself, with
# an exact softmax, reaches a worst row relL1 of 2.09e-3 at gain 2 (CPU
# emulation of its rounding points at the model's shape), so rows are held to
# 3e-3; a reference lifted 14 above the row max gives ~1e-2 there.
ROW_TOL = 3e-3


def gain_inputs(w, gamma):
    inp = synth.make_inputs(w)
    for k in ("q_gamma", "k_gamma"):
        inp[k] = torch.full_like(inp[k], gamma)
    for k in ("q_beta", "k_beta"):
        inp[k] = torch.zeros_like(inp[k])
    return inp


def worst_row(y, ref):
    y = y.reshape(-1, ref.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    return float((np.abs(y - ref).sum(1) / np.abs(ref).sum(1)).max())


@pytest.mark.parametrize("gamma", [1.9, 1.95, 2.0, 2.05, 2.2])
def test_qk_gain_band_s24_global_full(gamma):
    w = W["s24"]
    inp = gain_inputs(w, gamma)
    log(f"[case] s24 global, QK-norm gain {gamma}, beta 0, full oracle")
    y = np64(run("global", w, to_dev(inp)))
    ref = oracle.global_attention(f64(inp["X"]), oracle_params(w, inp))
    m = assert_parity(y, ref, f"s24/global/gain{gamma}")
    wr = worst_row(y, ref)
    log(f"  relL1 {m['relL1']:.3e} max/max {m['max_over_max']:.3e} worst row relL1 {wr:.3e}")
    assert wr <= ROW_TOL, wr


@pytest.mark.parametrize("gamma", [1.9, 2.0, 2.05, 2.2])
def test_qk_gain_band_s100_sampled(gamma):
    w = W["s100"]
    inp = gain_inputs(w, gamma)
    log(f"[case] s100 global, QK-norm gain {gamma}, beta 0, sampled rows")
    y = np64(run("global", w, to_dev(inp))).reshape(-1, w.d)
    rows = synth.sample_rows(w, 384).numpy()
    ref = oracle.global_attention_rows(f64(inp["X"]), oracle_params(w, inp), rows)
    m = assert_parity(y[rows], ref, f"s100/global/gain{gamma}/sampled")
    wr = worst_row(y[rows], ref)
    log(f"  relL1 {m['relL1']:.3e} max/max {m['max_over_max']:.3e} worst row relL1 {wr:.3e}")
    assert wr <= ROW_TOL, wr


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------

def test_deterministic_bitwise():
    w = W["s24"]
    d = to_dev(synth.make_inputs(w))
    for mode in ("global", "frame", "register"):
        a = run(mode, w, d)
        b = run(mode, w, d)
        assert torch.equal(a, b), mode


def test_global_s1_equals_frame_bitwise():
    w = configs.custom("one", 1, 26, 39, 1024, 16, cid=21)
    d = to_dev(synth.make_inputs(w))
    assert torch.equal(run("global", w, d), run("frame", w, d))


def test_wo_linearity_bitwise():
    w = W["tiny"]
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    y1 = run("global", w, d)
    d2 = dict(d)
    d2["Wo"] = (d["Wo"].float() * 2).to(torch.bfloat16)
    y2 = run("global", w, d2)
    assert torch.equal(y2.float(), y1.float() * 2)


def test_global_frame_permutation():
    """No frame index in RoPE: permuting frames permutes the global output."""
    w = configs.custom("perm", 6, 26, 39, 1024, 16, cid=22)
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    a = run("global", w, d)
    dp = dict(d)
    dp["X"] = d["X"][perm.cuda()].contiguous()
    b = run("global", w, dp)
    ref = oracle.global_attention_rows(f64(inp["X"]), oracle_params(w, inp),
                                       synth.sample_rows(w, 128).numpy())
    assert_parity(np64(b), np64(a[perm.cuda()]), "perm")
    assert_parity(np64(a).reshape(-1, w.d)[synth.sample_rows(w, 128).numpy()], ref, "perm/oracle")


def test_frame_then_register_patch_rows_bitwise():
    """Frame block then register block: patch rows equal the frame output bit for bit,
    in place (Y == X) and out of place."""
    w = W["s500"]
    d = to_dev(synth.make_inputs(w))
    f = run("frame", w, d)
    r = run("register", w, d, X=f)
    assert torch.equal(r[:, 17:], f[:, 17:])
    f2 = f.clone()
    r2 = run("register", w, d, X=f2, Y=f2)
    assert torch.equal(r2, r)


def test_stages_equal_full_call():
    w = W["s24"]
    d = to_dev(synth.make_inputs(w))
    from vggt_global_attention_amd import api
    for mode in ("global", "frame", "register"):
        blk = api.Block(mode, d["X"], w.H, w.grid_h, w.grid_w)
        full = blk(d["X"], d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"], d["k_gamma"], d["k_beta"])
        Y = torch.empty_like(d["X"])
        if mode == "register":
            Y.copy_(d["X"])
        for st in (B.STAGE_PREP, B.STAGE_QKV, B.STAGE_CORE, B.STAGE_OUT):
            blk.stage(st, d["X"], d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"], d["k_gamma"],
                      d["k_beta"], Y)
        torch.cuda.synchronize()
        assert torch.equal(full, Y), mode


def test_error_leaves_output_untouched():
    w = W["tiny"]
    d = to_dev(synth.make_inputs(w))
    s = B.make_shape(w.S, w.T, w.d, w.H, w.grid_h, w.grid_w)
    Y = torch.full_like(d["X"], 7.0)
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    st = B.vggt_attn_global(s, d["X"].data_ptr(), d["Wqkv"].data_ptr(), d["Wo"].data_ptr(),
                            d["q_gamma"].data_ptr(), d["q_beta"].data_ptr(), d["k_gamma"].data_ptr(),
                            d["k_beta"].data_ptr(), Y.data_ptr(), ws.data_ptr(), ws.numel(), None)
    torch.cuda.synchronize()
    assert st == B.EWORKSPACE
    assert bool((Y == 7.0).all())


def test_large_magnitudes_range_guard():
    """X scaled by 2^16 (v would overflow fp16 unscaled) and Wo by 2^-10: the
    power-of-two range guards keep v, O and Wo inside fp16."""
    w = W["tiny"]
    inp = synth.make_inputs(w)
    big = dict(inp)
    big["X"] = (inp["X"].float() * 65536).to(torch.bfloat16)
    big["Wo"] = (inp["Wo"].float() / 1024).to(torch.bfloat16)
    y = run("global", w, to_dev(big))
    ref = oracle.global_attention(f64(big["X"]), oracle_params(w, big))
    assert_parity(np64(y), ref, "tiny/large")


def test_register_patch_copy_ordered_on_caller_stream():
    """Register mode with Y != X, called on a non-default stream: work queued
    on that stream right after the call sees every row of Y, the copied patch
    rows included."""
    w = W["s500"]
    d = to_dev(synth.make_inputs(w))
    blk = api.Block("register", d["X"], w.H, w.grid_h, w.grid_w)
    args = [d[k] for k in ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            Y = torch.full_like(d["X"], float("nan"))
            blk(*args, Y=Y, stream=s)
            same = torch.equal(Y[:, 17:], d["X"][:, 17:])  # queued on s, right behind the call
            assert same
    torch.cuda.synchronize()
