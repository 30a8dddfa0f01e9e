"""GPU parity of the bf16-operand variant (vggt_attn_bf16ops: q, k, v, P, O
and the Wo copy in bf16, bf16 x bf16 MFMA, fp32 accumulation) against the
fp64 oracle, at its own bar (helpers.BF16OPS_*: the cost of bf16 rounding,
derived in test_precision_budget), for the frame, global and register
blocks; plus its stages against its full call, and a check that it is a
different computation from the default fp16-operand path."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from vggt_global_attention_amd import api, configs, synth
from vggt_global_attention_amd import binding as B
from helpers import (BF16OPS_MAX, BF16OPS_MEAN, BF16OPS_RELL1, f64, metrics,
                     oracle_params)
from gpu_common import log, np64, require_gpu, run, to_dev

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def check(y, ref, label):
    m = metrics(y, ref)
    log(f"  {label}: {m}")
    assert m["nonfinite"] == 0, m
    assert m["relL1"] <= BF16OPS_RELL1, m
    assert m["max_over_max"] <= BF16OPS_MAX, m
    assert m["mean_over_max"] <= BF16OPS_MEAN, m
    return m


ORACLE = {"frame": oracle.frame_attention, "global": oracle.global_attention,
          "register": oracle.register_attention}


@pytest.mark.parametrize("name,mode", [("tiny", "frame"), ("tiny", "global"), ("tiny", "register"),
                                       ("s24", "global"), ("s24", "frame")])
def test_full_oracle(name, mode):
    w = W[name]
    inp = synth.make_inputs(w)
    log(f"[case] bf16 operands {name} {mode}, full oracle")
    y = np64(run(mode, w, to_dev(inp), operands="bf16"))
    ref = ORACLE[mode](f64(inp["X"]), oracle_params(w, inp))
    check(y, ref, f"{name}/{mode}/bf16ops")


def test_ragged_register_and_frame():
    w = configs.custom("bf16_ragged", 5, 3, 7, 128, 2, cid=95)
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    X, p = f64(inp["X"]), oracle_params(w, inp)
    for mode in ("frame", "global", "register"):
        log(f"[case] bf16 operands ragged {mode}")
        check(np64(run(mode, w, d, operands="bf16")), ORACLE[mode](X, p), f"ragged/{mode}/bf16ops")


def test_s100_sampled_rows():
    w = W["s100"]
    inp = synth.make_inputs(w)
    log("[case] bf16 operands s100 global, sampled rows")
    y = np64(run("global", w, to_dev(inp), operands="bf16")).reshape(-1, w.d)
    rows = synth.sample_rows(w, 256).numpy()
    ref = oracle.global_attention_rows(f64(inp["X"]), oracle_params(w, inp), rows)
    check(y[rows], ref, "s100/global/bf16ops/sampled")


def test_stages_equal_call_and_differ_from_fp16():
    w = W["s24"]
    d = to_dev(synth.make_inputs(w))
    args = [d[k] for k in ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")]
    blk = api.Block("global", d["X"], w.H, w.grid_h, w.grid_w, operands="bf16")
    a = blk(*args).clone()
    Y = torch.empty_like(a)
    for st in (B.STAGE_PREP, B.STAGE_QKV, B.STAGE_CORE, B.STAGE_OUT):
        blk.stage(st, *args, Y)
    torch.cuda.synchronize()
    assert torch.equal(Y, a)
    f = run("global", w, d)
    assert not torch.equal(a, f)
    # same block, two roundings: the two results agree to the bf16 variant's bar
    m = metrics(np64(a), np64(f))
    log(f"  bf16 vs fp16 operands: {m}")
    assert m["relL1"] <= BF16OPS_RELL1, m


def test_rejects_other_modes():
    w = W["tiny"]
    d = to_dev(synth.make_inputs(w))
    with pytest.raises(ValueError):
        api.Block("subsampled", d["X"], w.H, w.grid_h, w.grid_w, operands="bf16")
