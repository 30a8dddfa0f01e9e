"""GPU checks of the split attention tail.

The last round of workgroups of a single-set grid (global sets, query
windows, subsampled and register sets) is only partly filled. The library
runs each of those workgroups as P key ranges. A merge kernel then combines
the ranges' softmax states.

What is checked:
- split results match the fp64 oracle at the block bar;
- they stay within a few fp16 roundings of O of the unsplit kernel
  (VGGT_ATTN_SPLIT = 1, through the tuning build);
- splitting every workgroup, forced splits, query windows and the 4-wave
  register grid are exercised.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from vggt_global_attention_amd import api, configs, synth
from helpers import assert_parity, f64, metrics, oracle_params
from gpu_common import log, np64, require_gpu, run, to_dev, tuned

pytestmark = pytest.mark.gpu

# split vs unsplit: the merge reorders fp32 sums of O and l only
CLOSE_RELL1 = 5e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def with_split(monkeypatch, ways, fn):
    with tuned(monkeypatch, VGGT_ATTN_SPLIT=ways):
        return fn()


def tail_rows(w, qtiles_per_head, n_tail, bq=512, count=64, seed=0):
    """Query rows whose last head runs in the split tail: the last n_tail
    workgroups are the last query tiles of the last head(s)."""
    first_tile = max(0, qtiles_per_head - n_tail)
    lo, hi = first_tile * bq, w.N
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(np.arange(lo, hi), min(count, hi - lo), replace=False))


@pytest.mark.parametrize("ways", [2, 3, 7, 16])
def test_forced_split_s24(monkeypatch, ways):
    """24 frames (784 workgroups): forced key ranges per split workgroup
    against the unsplit kernel and, on rows of the split tail, the oracle."""
    w = configs.WORKLOADS["s24"]
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    log(f"[case] s24 global, split {ways} ways vs unsplit")
    y1 = with_split(monkeypatch, 1, lambda: run("global", w, d))
    yp = with_split(monkeypatch, ways, lambda: run("global", w, d))
    m = metrics(np64(yp), np64(y1))
    assert m["relL1"] <= CLOSE_RELL1, m
    qt = -(-w.N // 512)
    n_tail = (qt * w.H) % cus()
    rows = tail_rows(w, qt, n_tail)
    ref = oracle.global_attention_rows(f64(inp["X"]), oracle_params(w, inp), rows)
    assert_parity(np64(yp.reshape(-1, w.d))[rows], ref, f"s24 split {ways}")


def test_split_every_workgroup(monkeypatch):
    """Three frames on the 8-wave tile (forced: a grid this small picks the
    4-wave one): 112 workgroups, fewer than the CUs, so the plan splits all
    of them (no whole workgroup); full oracle."""
    w = configs.custom("split3", 3, 26, 39, 1024, 16, cid=23)
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    with tuned(monkeypatch, VGGT_ATTN_WAVES=8):
        y = run("global", w, d)
    ref = oracle.global_attention(f64(inp["X"]), oracle_params(w, inp), threads=8)
    assert_parity(np64(y), ref, "3 frames, all split")


def test_split_ragged_keys(monkeypatch):
    """Four frames (4,124 keys: 64 full tiles and a 28-key tail) forced into
    two ranges: the masked tile is only in the last range."""
    w = configs.custom("split4", 4, 26, 39, 1024, 16, cid=24)
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    y1 = with_split(monkeypatch, 1, lambda: run("global", w, d))
    y2 = with_split(monkeypatch, 2, lambda: run("global", w, d))
    m = metrics(np64(y2), np64(y1))
    assert m["relL1"] <= CLOSE_RELL1, m
    ref = oracle.global_attention(f64(inp["X"]), oracle_params(w, inp), threads=8)
    assert_parity(np64(y2), ref, "4 frames, split 2")


def test_split_query_window(monkeypatch):
    """Query rows [1000, 4000) of 24 frames (96 workgroups): every workgroup
    split, the window offset carried into the merge."""
    w = configs.WORKLOADS["s24"]
    inp = synth.make_inputs(w)
    d = to_dev(inp)

    def call():
        blk = api.RowsBlock(d["X"], w.H, w.grid_h, w.grid_w, 1000, 3000)
        y = blk(*[d[k] for k in ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")])
        torch.cuda.synchronize()
        return y

    y = call()
    y1 = with_split(monkeypatch, 1, call)
    m = metrics(np64(y), np64(y1))
    assert m["relL1"] <= CLOSE_RELL1, m
    rows = np.sort(np.random.default_rng(3).choice(3000, 64, replace=False)) + 1000
    ref = oracle.global_attention_rows(f64(inp["X"]), oracle_params(w, inp), rows)
    assert_parity(np64(y)[rows - 1000], ref, "s24 rows window, split")


def test_split_register_s500(monkeypatch):
    """The 8,500-row register set of 500 frames on 4-wave workgroups of 64
    queries per wave (544 of them): split as planned against the unsplit
    kernel and the oracle."""
    w = configs.WORKLOADS["s500"]
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    y = run("register", w, d)
    y1 = with_split(monkeypatch, 1, lambda: run("register", w, d))
    spec = np.s_[:, :17]
    m = metrics(np64(y[spec]), np64(y1[spec]))
    assert m["relL1"] <= CLOSE_RELL1, m
    assert torch.equal(y[:, 17:], y1[:, 17:])
    frames = np.arange(0, w.S, 25)
    ref = oracle.register_attention(f64(inp["X"]), oracle_params(w, inp), threads=8)
    assert_parity(np64(y[frames, :17]), ref[frames, :17], "s500 register, split")


def test_split_subsampled_s24(monkeypatch):
    """Subsampled global set of 24 frames with 3 x 3 windows (3,216 kept keys):
    two key ranges per tail workgroup; the diagonal and mean columns enter in
    the last range only."""
    from oracle import avggt_sga
    w = configs.WORKLOADS["s24"]
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    y1 = with_split(monkeypatch, 1, lambda: run("subsampled", w, d, sub=(3, 3)))
    y2 = with_split(monkeypatch, 2, lambda: run("subsampled", w, d, sub=(3, 3)))
    m = metrics(np64(y2), np64(y1))
    assert m["relL1"] <= CLOSE_RELL1, m
    qt = -(-w.N // 512)
    rows = tail_rows(w, qt, (qt * w.H) % cus())
    ref = avggt_sga.sga_attention_rows(f64(inp["X"]), oracle_params(w, inp), 3, 3, rows)
    assert_parity(np64(y2.reshape(-1, w.d))[rows], ref, "s24 subsampled split 2")
