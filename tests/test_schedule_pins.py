"""Pins for the fp64 oracle of the attention-only layer schedule.

Each check ties `oracle.schedule` to something other than itself: the layer
indices the explainer page prints (tests/golden/aggregator_schedule.json),
torch's bf16 rounding, identities that follow from the definitions (a global
set of one frame is that frame's set; a residual layer with a zero branch is
the identity; frames that never meet stay independent), and planted mistakes
the pins must catch.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import schedule as sg
from oracle.vggt_oracle import OracleParams
from vggt_global_attention_amd import schedule as pkg_schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "aggregator_schedule.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def make_blocks(n_blocks, d=32, H=2, gh=2, gw=3, seed=0, ls=0.3):
    rng = np.random.default_rng(seed)
    blocks, scales = [], []
    for _ in range(n_blocks):
        blocks.append(OracleParams(
            Wqkv=rng.standard_normal((3 * d, d)) / math.sqrt(d),
            Wo=rng.standard_normal((d, d)) / math.sqrt(d),
            q_gamma=1 + 0.3 * rng.standard_normal((H, d // H)),
            q_beta=0.3 * rng.standard_normal((H, d // H)),
            k_gamma=1 + 0.3 * rng.standard_normal((H, d // H)),
            k_beta=0.3 * rng.standard_normal((H, d // H)),
            H=H, grid_h=gh, grid_w=gw))
        scales.append(ls * (1 + 0.1 * rng.standard_normal(d)))
    return blocks, scales


def make_x(S, d=32, gh=2, gw=3, seed=1):
    rng = np.random.default_rng(seed)
    return sg.round_bf16(rng.standard_normal((S, 17 + gh * gw, d)))


# ----------------------------------------------------------------------------
# Pins
# ----------------------------------------------------------------------------

def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(37.0)
    # exact ties: a bf16 value plus half its unit in the last place
    b = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    m, e = np.frexp(b.astype(np.float64))
    ties = (b.astype(np.float64) + np.ldexp(1.0, e - 9)).astype(np.float32)
    vals = np.concatenate([x, ties, -ties, np.float32([0.0, 1.0, -2.5, 3.0e-30, 6.0e30])])
    ref = torch.tensor(vals).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(sg.round_bf16(vals.astype(np.float64)), ref)


def test_layer_constants_are_the_pages():
    g = golden()
    spec = sg.Spec()
    assert spec.n_layers == g["n_layers"]
    assert tuple(spec.register_layers) == tuple(g["register_layers"])
    assert tuple(spec.cached_layers) == tuple(g["cached_layers"])
    assert sg.N_SPECIAL == g["special_tokens_per_frame"]
    # the library front end carries the same schedule
    p = pkg_schedule.ScheduleSpec()
    assert (p.n_layers, tuple(p.register_layers), tuple(p.cached_layers)) == \
        (g["n_layers"], tuple(g["register_layers"]), tuple(g["cached_layers"]))
    assert all(p.inter_mode(l) == spec.inter_mode(l) for l in range(24))


def _register_pin(runner=None):
    """Patch rows change in the inter-frame block exactly outside the page's
    register layers; special rows change in every block."""
    runner = runner or sg.run_schedule
    g = golden()
    blocks, scales = make_blocks(48, seed=5)
    X = make_x(2, seed=6)
    _, _, states = runner(X, blocks, scales, sg.Spec(), threads=1, trace=True)
    prev = X
    for l, (a, x) in enumerate(states):
        assert not np.array_equal(a[:, 17:], prev[:, 17:]), l       # frame block, patches
        assert not np.array_equal(x[:, :17], a[:, :17]), l          # inter block, specials
        patches_same = np.array_equal(x[:, 17:], a[:, 17:])
        assert patches_same == (l in g["register_layers"]), l
        prev = x


def test_register_layers_leave_patches():
    _register_pin()


def _cache_pin(runner=None):
    runner = runner or sg.run_schedule
    g = golden()
    blocks, scales = make_blocks(48, seed=7)
    X = make_x(2, seed=8)
    state, caches, states = runner(X, blocks, scales, sg.Spec(), threads=1, trace=True)
    assert caches.shape == (4, 2, 23, 64)
    for k, l in enumerate(g["cached_layers"]):
        np.testing.assert_array_equal(caches[k][..., :32], states[l][0])
        np.testing.assert_array_equal(caches[k][..., 32:], states[l][1])
    np.testing.assert_array_equal(state, states[-1][1])


def test_caches_are_the_kept_states():
    _cache_pin()


def _sequential_pin(runner=None):
    """With one frame, a global block is the frame block of the same weights.
    One layer [frame W, inter W] then equals two layers [frame W, inter with a
    zero branch] twice: the inter-frame block must act on the state the frame
    block left, not on the layer's input."""
    runner = runner or sg.run_schedule
    blocks, scales = make_blocks(1, seed=9)
    W, ls = blocks[0], scales[0]
    X = make_x(1, seed=10)
    zero = np.zeros_like(ls)
    spec1 = sg.Spec(n_layers=1, register_layers=(), cached_layers=())
    spec2 = sg.Spec(n_layers=2, register_layers=(), cached_layers=())
    one, _ = runner(X, [W, W], [ls, ls], spec1, threads=1)
    two, _ = runner(X, [W, W, W, W], [ls, zero, ls, zero], spec2, threads=1)
    np.testing.assert_array_equal(one, two)


def test_inter_block_follows_frame_block():
    _sequential_pin()


def test_zero_branches_are_identity():
    blocks, scales = make_blocks(8, seed=11)
    X = make_x(2, seed=12)
    spec = sg.Spec(n_layers=4, register_layers=(1,), cached_layers=(0, 3))
    state, caches = sg.run_schedule(X, blocks, [np.zeros_like(s) for s in scales], spec, threads=1)
    np.testing.assert_array_equal(state, X)
    for c in caches:
        np.testing.assert_array_equal(c, np.concatenate([X, X], axis=-1))


def test_all_frame_layers_keep_frames_independent():
    # AVGGT's conversion applied to every layer (and no register layer): no
    # block ever mixes frames, so each frame evolves on its own.
    blocks, scales = make_blocks(12, seed=13)
    X = make_x(3, seed=14)
    spec = sg.Spec(n_layers=6, register_layers=(), cached_layers=(2,), early_frame=6)
    state, caches = sg.run_schedule(X, blocks, scales, spec, threads=1)
    for s in range(3):
        one, c1 = sg.run_schedule(X[s:s + 1], blocks, scales, spec, threads=1)
        np.testing.assert_array_equal(state[s:s + 1], one)
        np.testing.assert_array_equal(caches[:, s:s + 1], c1)
    # and the global schedule does mix them
    g, _ = sg.run_schedule(X, blocks, scales, sg.Spec(n_layers=6, register_layers=(),
                                                      cached_layers=()), threads=1)
    assert not np.array_equal(g, state)


def test_subsampled_schedule_with_unit_windows_is_global():
    blocks, scales = make_blocks(6, seed=15)
    X = make_x(2, seed=16)
    base = dict(n_layers=3, register_layers=(1,), cached_layers=(0, 2))
    a = sg.run_schedule(X, blocks, scales, sg.Spec(**base), threads=1)
    # sub=(1,1) keeps every key: the subsampled block is the global block
    spec = sg.Spec(**base)
    b_blocks = [sg.inter_block(X, blocks[1], "subsampled", (1, 1), threads=1),
                sg.inter_block(X, blocks[1], "global", None, threads=1)]
    np.testing.assert_allclose(b_blocks[0], b_blocks[1], rtol=0, atol=1e-12)
    assert spec.inter_mode(0) == "global" and spec.inter_mode(1) == "register"
    assert sg.Spec(**base, sub=(2, 2)).inter_mode(0) == "subsampled"
    assert sg.Spec(**base, early_frame=1, sub=(2, 2)).inter_mode(0) == "frame"
    assert a[0].shape == X.shape


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_mutation_one_based_register_layers(monkeypatch):
    orig = sg.Spec.inter_mode

    def shifted(self, l):
        return orig(sg.Spec(self.n_layers, tuple(i - 1 for i in self.register_layers),
                            self.cached_layers, self.early_frame, self.sub), l)
    monkeypatch.setattr(sg.Spec, "inter_mode", shifted)
    assert _fails(_register_pin)


def _mutated_runner(kind):
    def run(X, blocks, layer_scales, spec, threads=None, trace=False):
        x = np.asarray(X, dtype=np.float64)
        special = (np.arange(x.shape[1]) < 17)[None, :, None]
        caches, states = [], []
        for l in range(spec.n_layers):
            y = sg.round_bf16(sg.frame_attention(x, blocks[2 * l], threads))
            a = sg.round_bf16(x + layer_scales[2 * l] * y)
            mode = spec.inter_mode(l)
            src = x if kind == "parallel" else a
            y = sg.round_bf16(sg.inter_block(src, blocks[2 * l + 1], mode, spec.sub, threads))
            upd = sg.round_bf16(a + layer_scales[2 * l + 1] * y)
            if kind == "register_all_rows":
                x = upd
            else:
                x = np.where(special, upd, a) if mode == "register" else upd
            if l in spec.cached_layers:
                pair = [x, a] if kind == "cache_order" else [a, x]
                caches.append(np.concatenate(pair, axis=-1))
            states.append((a, x))
        caches = np.stack(caches) if caches else np.zeros((0,))
        return (x, caches, states) if trace else (x, caches)
    return run


def test_mutation_parallel_branches():
    assert _fails(_sequential_pin, _mutated_runner("parallel"))


def test_mutation_register_updates_patches():
    assert _fails(_register_pin, _mutated_runner("register_all_rows"))


def test_mutation_cache_order():
    assert _fails(_cache_pin, _mutated_runner("cache_order"))


def test_unmutated_runner_passes_every_pin():
    # the mutation harness itself is faithful when nothing is planted
    r = _mutated_runner("none")
    _register_pin(r)
    _cache_pin(r)
    _sequential_pin(r)


def test_perturb_hook_identity_is_the_composition():
    """The perturbation hook (for deriving how far per-block errors carry)
    changes nothing when it returns its input, and does change the result
    when it scales a block."""
    blocks, scales = make_blocks(6, seed=9)
    X = make_x(2, seed=10)
    spec = sg.Spec(n_layers=3, register_layers=(1,), cached_layers=(0, 2))
    ref, c0 = sg.run_schedule(X, blocks, scales, spec, threads=1)
    same, c1 = sg.run_schedule(X, blocks, scales, spec, threads=1, perturb=lambda y, b: y)
    assert np.array_equal(ref, same) and np.array_equal(c0, c1)
    other, _ = sg.run_schedule(X, blocks, scales, spec, threads=1,
                               perturb=lambda y, b: y * (2.0 if b == 4 else 1.0))
    assert not np.array_equal(ref, other)


def test_merging_with_r0_is_the_plain_schedule():
    """HTTM merging in the global inter-frame blocks with r = 0 merges nothing:
    the composition is exactly the plain one; with r > 0 it differs."""
    blocks, scales = make_blocks(8, seed=11, gh=2, gw=3)
    X = make_x(4, seed=12)
    spec = sg.Spec(n_layers=4, register_layers=(1,), cached_layers=(3,))
    ref, c0 = sg.run_schedule(X, blocks, scales, spec, threads=1)
    same, c1 = sg.run_schedule(X, blocks, scales,
                               sg.Spec(n_layers=4, register_layers=(1,), cached_layers=(3,),
                                       merge=(2, 1, 2, 0)), threads=1)
    assert np.array_equal(ref, same) and np.array_equal(c0, c1)
    merged, _ = sg.run_schedule(X, blocks, scales,
                                sg.Spec(n_layers=4, register_layers=(1,), cached_layers=(3,),
                                        merge=(2, 1, 2, 2)), threads=1)
    assert not np.array_equal(ref, merged)
    assert [sg.Spec(n_layers=4, register_layers=(1,), merge=(2, 1, 2, 2)).inter_mode(l)
            for l in range(4)] == ["merged", "register", "merged", "merged"]
