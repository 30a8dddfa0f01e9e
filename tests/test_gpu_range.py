"""GPU checks of the device-side value-range status (VGGT_ATTN_RANGE_* bits,
read with vggt_attn_range_status after the call).

A call's prep stage flags non-finite inputs, QK-norm affines that could
overflow fp16 q / k, and bounds that the power-of-two pre-scales of v, O and
Wo cannot bring into fp16 range -- the inputs for which Y may hold inf or
NaN -- without any host synchronisation.  The kernels still run to the end on
such inputs (only fp16 / bf16 overflow and NaN propagation happen, no access
depends on a value), so every case here is a normal launch.
"""

from __future__ import annotations

import pytest
import torch

from vggt_global_attention_amd import api, configs, synth
from vggt_global_attention_amd import binding as B
from vggt_global_attention_amd import schedule as S
from vggt_global_attention_amd.descriptor import DescriptorCache
from gpu_common import log, require_gpu, to_dev

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS["tiny"]
KEYS = ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def call(mode, d):
    blk = api.Block(mode, d["X"], W.H, W.grid_h, W.grid_w)
    y = blk(*[d[k] for k in KEYS])
    st, bits = B.vggt_attn_range_status(blk.workspace.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return y, st, bits


def base():
    return to_dev(synth.make_inputs(W))


@pytest.mark.parametrize("mode", ["frame", "global", "register"])
def test_in_range_inputs_report_ok(mode):
    y, st, bits = call(mode, base())
    assert (st, bits) == (B.OK, 0)
    assert bool(torch.isfinite(y.float()).all())


def _with(name, fn):
    d = base()
    d[name] = fn(d[name].clone())
    return d


def _set(t, idx, v):
    t.view(-1)[idx] = v
    return t


NAN, INF = float("nan"), float("inf")
CASES = [
    ("X NaN", lambda: _with("X", lambda t: _set(t, 12345, NAN)), B.RANGE_X),
    ("X inf", lambda: _with("X", lambda t: _set(t, 7, INF)), B.RANGE_X),
    # row norms beyond fp32: |x| ~ 2^70, squared 2^140
    ("X 2^70", lambda: _with("X", lambda t: (t.float() * 2.0 ** 70).to(torch.bfloat16)), B.RANGE_X),
    ("Wq NaN", lambda: _with("Wqkv", lambda t: _set(t, 3, NAN)), B.RANGE_WQKV),
    ("Wk NaN", lambda: _with("Wqkv", lambda t: _set(t, W.d * W.d + 5, NAN)), B.RANGE_WQKV),
    ("Wv inf", lambda: _with("Wqkv", lambda t: _set(t, 2 * W.d * W.d + 9, -INF)), B.RANGE_WQKV),
    ("Wo NaN", lambda: _with("Wo", lambda t: _set(t, 100, NAN)), B.RANGE_WO),
    ("k gamma 1e5", lambda: _with("k_gamma", lambda t: t.fill_(1e5)), B.RANGE_AFFINE),
    ("q beta NaN", lambda: _with("q_beta", lambda t: _set(t, 0, NAN)), B.RANGE_AFFINE),
]


@pytest.mark.parametrize("label,make,bit", CASES, ids=[c[0] for c in CASES])
def test_flagged_inputs(label, make, bit):
    log(f"[case] range status: {label}")
    for mode in ("global", "frame"):
        _, st, bits = call(mode, make())
        assert st == B.ERANGE and bits & bit, (label, mode, st, bits)


def test_value_bound_past_the_scale_clamp():
    """X scaled by 2^50 and the V rows of Wqkv by 2^30: max||x|| max||w_v|| ~
    2^85 needs a pre-scale of 2^-71, past the 2^-60 the scales are held to
    (v would overflow fp16).  Finite inputs, so only the scale bit."""
    d = base()
    d["X"] = (d["X"].float() * 2.0 ** 50).to(torch.bfloat16)
    Wqkv = d["Wqkv"].clone()
    Wqkv[2 * W.d:] = (Wqkv[2 * W.d:].float() * 2.0 ** 30).to(torch.bfloat16)
    d["Wqkv"] = Wqkv
    for mode in ("global", "frame", "register"):
        _, st, bits = call(mode, d)
        assert (st, bits) == (B.ERANGE, B.RANGE_SCALE), (mode, st, bits)


def test_large_but_reachable_magnitudes_stay_ok():
    """X by 2^16 and Wo by 2^-10 (the range-guard parity case) are inside the
    scales' reach: no bit."""
    d = base()
    d["X"] = (d["X"].float() * 65536).to(torch.bfloat16)
    d["Wo"] = (d["Wo"].float() / 1024).to(torch.bfloat16)
    _, st, bits = call("global", d)
    assert (st, bits) == (B.OK, 0)


def test_status_is_per_call():
    """A flagged call followed by a clean one on the same workspace: the second
    call's prep stage replaces the word."""
    bad = _with("Wo", lambda t: _set(t, 1, NAN))
    good = base()
    blk = api.Block("global", good["X"], W.H, W.grid_h, W.grid_w)
    s = torch.cuda.current_stream().cuda_stream
    blk(*[bad[k] for k in KEYS])
    assert B.vggt_attn_range_status(blk.workspace.data_ptr(), s) == (B.ERANGE, B.RANGE_WO)
    blk(*[good[k] for k in KEYS])
    assert B.vggt_attn_range_status(blk.workspace.data_ptr(), s) == (B.OK, 0)


def test_descriptor_attend_flags_a_nonfinite_descriptor():
    d = base()
    cache = DescriptorCache(W.d, W.H, 64)
    D = synth.make_descriptors(W, 40).cuda()
    cache.append(D, d["Wqkv"], d["k_gamma"], d["k_beta"])
    cache.attend(d["X"], W.grid_h, W.grid_w, d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"])
    s = torch.cuda.current_stream().cuda_stream
    assert B.vggt_attn_range_status(cache._ws.data_ptr(), s) == (B.OK, 0)
    D2 = synth.make_descriptors(W, 8, 1).cuda()
    D2[3, 5] = float("nan")
    cache.append(D2, d["Wqkv"], d["k_gamma"], d["k_beta"])
    cache.attend(d["X"], W.grid_h, W.grid_w, d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"])
    st, bits = B.vggt_attn_range_status(cache._ws.data_ptr(), s)
    assert st == B.ERANGE and bits & B.RANGE_X, (st, bits)


def test_schedule_accumulates_over_blocks():
    """A 4-layer schedule whose block 5 (layer 2's inter-frame block) has a
    non-finite Wo: the schedule's status word ORs every block's bits, so the
    flag survives the later blocks -- which also flag their input state, made
    non-finite by that block's output."""
    w = configs.custom("range_sched", S=2, grid_h=3, grid_w=4, d=128, H=2, cid=71)
    cpu = synth.make_block_weights(w, 8, 0.25)
    dev = [{k: v.cuda().contiguous() for k, v in b.items()} for b in cpu]
    X = synth.make_inputs(w)["X"].cuda()
    spec = S.ScheduleSpec(n_layers=4, register_layers=(1,), cached_layers=())
    sch = S.Schedule(X, w.H, w.grid_h, w.grid_w, dev, spec)
    s = torch.cuda.current_stream().cuda_stream
    sch(X)
    assert B.vggt_attn_range_status(sch.workspace.data_ptr(), s) == (B.OK, 0)
    dev[5]["Wo"] = dev[5]["Wo"].clone()
    dev[5]["Wo"].view(-1)[17] = NAN
    sch2 = S.Schedule(X, w.H, w.grid_h, w.grid_w, dev, spec, workspace=sch.workspace)
    sch2(X)
    assert B.vggt_attn_range_status(sch.workspace.data_ptr(), s) == \
        (B.ERANGE, B.RANGE_WO | B.RANGE_X)
    # only the last block bad: its own bit, no X bit (its input state is clean)
    dev[5]["Wo"] = cpu[5]["Wo"].cuda().contiguous()
    dev[7]["Wo"] = dev[7]["Wo"].clone()
    dev[7]["Wo"].view(-1)[3] = NAN
    S.Schedule(X, w.H, w.grid_h, w.grid_w, dev, spec, workspace=sch.workspace)(X)
    assert B.vggt_attn_range_status(sch.workspace.data_ptr(), s) == (B.ERANGE, B.RANGE_WO)
