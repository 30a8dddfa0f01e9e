"""GPU checks of the layer schedule (vggt_attn_schedule_run) and the residual
update (vggt_attn_residual) against their definitions and the fp64 oracle.

Bars:
* Residual update: the definition is z = bf16(fp32 fma(gamma, y, x)).  The
  reference computes x + gamma * y in float64 (exact for these operands) and
  rounds to fp32, then to bf16; both sides must agree bit for bit.
* One schedule block: given the GPU's own input state (every layer kept, so
  every block's input is known), the oracle's block output y_ref gives the
  next state ref = bf16(a + gamma * bf16(y_ref)).  The GPU's block output is
  within the block bar (max error <= 1e-2 * max|y_ref|), so before rounding
  the two next states differ by at most max(gamma) * 1e-2 * max|y_ref| (plus
  the bf16 rounding of y, inside that bar); rounding each to bf16 adds at most
  one unit in the last place of the result.  That bound is checked element by
  element, and the relL1 of the branch (next state - input) to the block bar
  scaled by the rounding noise.
* End to end, the final state against the oracle's own composition: the
  per-block differences above do not simply add up -- a one-unit rounding
  flip in a bf16 state feeds every later block.  The bound is derived with
  the oracle: its composition with every block output perturbed at the
  block bar (elementwise relative noise, relL1 ~2e-3 per block) shows how
  far such errors carry through the layers (carried_error_bound); the GPU's
  final state must stay within 1.25x that relL1 and 2x that max/max.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import httm as ohttm
from oracle import schedule as osched
from oracle.vggt_oracle import OracleParams
from vggt_global_attention_amd import configs, synth
from vggt_global_attention_amd import schedule as S
from helpers import f64, metrics
from gpu_common import log, np64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def bf16_round_via_fp32(x64: np.ndarray) -> np.ndarray:
    return torch.tensor(x64, dtype=torch.float64).to(torch.float32).to(torch.bfloat16) \
        .to(torch.float64).numpy()


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 8)


# ----------------------------------------------------------------------------
# Residual update
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("rows,d,period,active", [(1000, 256, 1, 1), (37 * 5, 128, 37, 17),
                                                  (3, 1024, 1, 1), (4096, 64, 64, 1)])
def test_residual_definition(rows, d, period, active):
    log(f"[case] residual rows={rows} d={d} period={period} active={active}")
    g = torch.Generator().manual_seed(rows + d)
    X = torch.randn(rows, d, generator=g).to(torch.bfloat16)
    Y = (3 * torch.randn(rows, d, generator=g)).to(torch.bfloat16)
    gamma = torch.randn(d, generator=g) * 0.3
    Xd, Yd, gd = X.cuda(), Y.cuda(), gamma.cuda()
    C = torch.full((rows, 2 * d), 7.0, dtype=torch.bfloat16, device="cuda")
    Z = S.residual(Xd, Yd, gd, period=period, active=active, C=C[:, d:], c_stride=2 * d)
    torch.cuda.synchronize()
    x, y, gm = f64(X), f64(Y), f64(gamma)
    ref = bf16_round_via_fp32(x + gm[None, :] * y)
    on = (np.arange(rows) % period < active)[:, None]
    ref = np.where(on, ref, x)
    np.testing.assert_array_equal(np64(Z), ref)
    np.testing.assert_array_equal(np64(C[:, d:]), ref)
    assert bool((C[:, :d] == 7.0).all())          # the other half is untouched
    # in place
    Xi = Xd.clone()
    S.residual(Xi, Yd, gd, Z=Xi, period=period, active=active)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np64(Xi), ref)


# ----------------------------------------------------------------------------
# Schedule
# ----------------------------------------------------------------------------

def block_weights(w, n_blocks, ls):
    cpu = synth.make_block_weights(w, n_blocks, ls)
    dev = [{k: v.cuda().contiguous() for k, v in b.items()} for b in cpu]
    params = [OracleParams(Wqkv=f64(b["Wqkv"]), Wo=f64(b["Wo"]), q_gamma=f64(b["q_gamma"]),
                           q_beta=f64(b["q_beta"]), k_gamma=f64(b["k_gamma"]),
                           k_beta=f64(b["k_beta"]), H=w.H, grid_h=w.grid_h, grid_w=w.grid_w,
                           rope_base=w.rope_base, ln_eps=w.ln_eps) for b in cpu]
    scales = [f64(b["layer_scale"]) for b in cpu]
    return dev, params, scales


def local_block_checks(X, states_gpu, params, scales, spec, label):
    """Every block of the GPU run against the oracle block on the GPU's own
    input state (see the module docstring for the bound)."""
    prev = X
    T = X.shape[1]
    special = (np.arange(T) < 17)[None, :, None]
    worst = 0.0
    for l, (a_g, x_g) in enumerate(states_gpu):
        for half, (inp, out, mode) in enumerate(((prev, a_g, "frame"),
                                                 (a_g, x_g, spec.inter_mode(l)))):
            p, gam = params[2 * l + half], scales[2 * l + half]
            y = osched.round_bf16(osched.inter_block(inp, p, mode, spec.params(mode)))
            ref = osched.round_bf16(inp + gam * y)
            if mode == "register":
                ref = np.where(special, ref, inp)
                y = np.where(special, y, 0.0)
            # merged blocks: tokens whose merge decision in some head is a
            # near-tie (oracle.httm.fragile) may take the other, equally valid
            # choice; they are left out of this block's check
            keep = np.ones(inp.shape[:2], dtype=bool)
            if mode == "merged":
                frag = ohttm.fragile(inp, p, ohttm.HttmParams(*spec.merge)).any(axis=1)
                keep = ~frag.reshape(inp.shape[:2])
            bound = np.abs(gam).max() * 1e-2 * np.abs(y).max() + ulp_bf16(ref)
            err = np.abs(out - ref)
            bad = (err > bound) & keep[..., None]
            assert not bad.any(), (label, l, half, mode, float((err - bound)[bad].max()))
            m = metrics((out - inp)[keep], (ref - inp)[keep])
            worst = max(worst, m["relL1"])
            # the branch itself: the block bar plus the bf16 rounding of both states
            noise = float(np.mean(ulp_bf16(ref) / 2) / max(np.mean(np.abs(ref - inp)), 1e-30))
            assert m["relL1"] <= 2e-3 + noise, (label, l, half, mode, m, noise)
        prev = x_g
    log(f"  {label}: worst branch relL1 {worst:.2e}")


def run_gpu(w, dev_blocks, spec, X):
    Xd = X.cuda()
    sch = S.Schedule(Xd, w.H, w.grid_h, w.grid_w, dev_blocks, spec)
    state, caches = sch(Xd)
    torch.cuda.synchronize()
    return state, caches


def split_caches(caches, d):
    c = np64(caches)
    return [(c[k][..., :d], c[k][..., d:]) for k in range(c.shape[0])]


def carried_error_bound(X, params, scales, spec, seeds=3, a=4e-3):
    """How far per-block errors at the block bar carry through the layers: the
    oracle's composition with every block output multiplied by 1 + u, u
    uniform in [-a, a] elementwise (a = 4e-3 gives each block relL1 ~2e-3,
    the block bar), against the unperturbed composition; the largest relL1
    and max/max over a few seeds.  Dominated by one-unit flips of the bf16
    state that every later block then sees."""
    ref, _ = osched.run_schedule(X, params, scales, spec)
    worst = {"relL1": 0.0, "max_over_max": 0.0}
    for seed in range(seeds):
        rng = np.random.default_rng(seed)
        st, _ = osched.run_schedule(
            X, params, scales, spec,
            perturb=lambda y, b: y * (1.0 + rng.uniform(-a, a, size=y.shape)))
        m = metrics(st, ref)
        for k in worst:
            worst[k] = max(worst[k], m[k])
    return ref, worst


SCHED_TINY = configs.custom("sched_tiny", S=3, grid_h=4, grid_w=5, d=128, H=2, cid=61)


def test_schedule_24_layers_tiny():
    w = SCHED_TINY
    log(f"[case] schedule 24 layers, S={w.S} T={w.T} d={w.d}")
    dev, params, scales = block_weights(w, 48, 0.25)
    X = synth.make_inputs(w)["X"]
    spec_all = S.ScheduleSpec(cached_layers=tuple(range(24)))
    state, caches = run_gpu(w, dev, spec_all, X)
    states = split_caches(caches, w.d)
    np.testing.assert_array_equal(states[-1][1], np64(state))
    ospec = osched.Spec(cached_layers=tuple(range(24)))
    local_block_checks(f64(X), states, params, scales, ospec, "24 layers")
    # end to end against the oracle's own composition, within what errors at
    # the block bar in every block produce through the 48 blocks (1.25x the
    # worst relL1 of the modelled compositions, 2x their max/max)
    ref, carried = carried_error_bound(f64(X), params, scales, osched.Spec())
    m = metrics(np64(state), ref)
    log(f"  end to end: {m}; block-bar errors carried through the layers: {carried}")
    assert m["nonfinite"] == 0
    assert m["relL1"] <= 1.25 * carried["relL1"], (m, carried)
    assert m["max_over_max"] <= 2.0 * carried["max_over_max"], (m, carried)
    # the page's schedule with its four kept layers, in place: bitwise the same
    Xd = X.cuda()
    sch = S.Schedule(Xd, w.H, w.grid_h, w.grid_w, dev)
    st2, c2 = sch(Xd, state=Xd)
    torch.cuda.synchronize()
    assert torch.equal(st2, state)
    for k, l in enumerate(osched.CACHED_LAYERS):
        assert torch.equal(c2[k], caches[l]), l


def test_schedule_with_merging():
    """Eight layers with HTTM merging in the global inter-frame blocks (runs
    of 2 frames, 2 x 2 windows, 2 merges per block) and two register
    layers: every block against the oracle block on the GPU's input state
    (near-tie tokens of merged blocks left out), and the final state within
    what block-bar errors carry through the layers."""
    w = configs.custom("sched_httm", S=4, grid_h=4, grid_w=5, d=128, H=2, cid=63)
    merge = (2, 2, 2, 2)
    spec = S.ScheduleSpec(n_layers=8, register_layers=(2, 6), cached_layers=tuple(range(8)),
                          merge=merge)
    log(f"[case] schedule with HTTM merging {merge}, 8 layers")
    dev, params, scales = block_weights(w, 16, 0.25)
    X = synth.make_inputs(w)["X"]
    state, caches = run_gpu(w, dev, spec, X)
    ospec = osched.Spec(n_layers=8, register_layers=(2, 6), cached_layers=tuple(range(8)),
                        merge=merge)
    assert [spec.inter_mode(l) for l in range(8)] == [ospec.inter_mode(l) for l in range(8)]
    assert spec.inter_mode(0) == "merged"
    local_block_checks(f64(X), split_caches(caches, w.d), params, scales, ospec, "httm")
    ref, carried = carried_error_bound(f64(X), params, scales, ospec)
    m = metrics(np64(state), ref)
    log(f"  end to end: {m}; block-bar errors carried through the layers: {carried}")
    assert m["nonfinite"] == 0
    assert m["relL1"] <= 1.25 * carried["relL1"], (m, carried)


def test_schedule_avggt_conversions():
    w = SCHED_TINY
    spec = S.ScheduleSpec(n_layers=8, register_layers=(2, 6), cached_layers=tuple(range(8)),
                          early_frame=3, sub=(2, 2))
    log(f"[case] schedule AVGGT early_frame=3 sub=2x2, 8 layers")
    dev, params, scales = block_weights(w, 16, 0.25)
    X = synth.make_inputs(w)["X"]
    state, caches = run_gpu(w, dev, spec, X)
    ospec = osched.Spec(n_layers=8, register_layers=(2, 6), cached_layers=tuple(range(8)),
                        early_frame=3, sub=(2, 2))
    assert [spec.inter_mode(l) for l in range(8)] == [ospec.inter_mode(l) for l in range(8)]
    local_block_checks(f64(X), split_caches(caches, w.d), params, scales, ospec, "avggt")


def test_schedule_real_width():
    """Four layers at the model's width and frame shape (d = 1024, 16 heads,
    26 x 39 patches), three frames; layer 2 is a register layer."""
    w = configs.custom("sched_real", S=3, grid_h=26, grid_w=39, d=1024, H=16, cid=62)
    spec = S.ScheduleSpec(n_layers=4, register_layers=(2,), cached_layers=(0, 1, 2, 3))
    log(f"[case] schedule real width, 4 layers, S={w.S} T={w.T}")
    dev, params, scales = block_weights(w, 8, 0.25)
    X = synth.make_inputs(w)["X"]
    state, caches = run_gpu(w, dev, spec, X)
    ospec = osched.Spec(n_layers=4, register_layers=(2,), cached_layers=(0, 1, 2, 3))
    local_block_checks(f64(X), split_caches(caches, w.d), params, scales, ospec, "real width")
