"""GPU parity of descriptor attention with a chunk-recursive cache
(vggt_attn_desc_*) against the fp64 oracle (`oracle.descriptor`), at the
block bar: max|err| <= 1e-2 * max|ref| and relL1 <= 2e-3."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import descriptor as odesc
from vggt_global_attention_amd import api, configs, synth
from vggt_global_attention_amd.descriptor import DescriptorCache
from helpers import assert_parity, f64, oracle_params
from gpu_common import log, np64, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def weights(d):
    return d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"], d["k_gamma"], d["k_beta"]


def attend(cache, w, d, X):
    Y = cache.attend(X, w.grid_h, w.grid_w, d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"])
    torch.cuda.synchronize()
    return Y


TINY = configs.custom("desc_tiny", S=4, grid_h=4, grid_w=5, d=128, H=2, cid=63)


@pytest.mark.parametrize("scale2", [1.0, 64.0])
def test_chunk_recursive_tiny(scale2):
    """Three chunks of frames with 37, 5 and 100 descriptors (ragged against
    the 16- and 64-key groups); scale2 = 64 makes the second chunk's norms
    jump, which lowers the cache's value exponent and rescales what is
    stored."""
    w = TINY
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    p = oracle_params(w, inp)
    Dc = [synth.make_descriptors(w, 37, 0), synth.make_descriptors(w, 5, 1, scale=scale2),
          synth.make_descriptors(w, 100, 2)]
    frames = [(0, 1), (1, 3), (3, 4)]
    cache = DescriptorCache(w.d, w.H, 200)
    X = inp["X"]
    for c, (a, b) in enumerate(frames):
        log(f"[case] descriptor tiny scale2={scale2} chunk {c}: frames {a}..{b - 1}, "
            f"{Dc[c].shape[0]} new descriptors")
        cache.append(Dc[c].cuda(), d["Wqkv"], d["k_gamma"], d["k_beta"])
        Xc = d["X"][a:b].contiguous()
        y = attend(cache, w, d, Xc)
        ref = odesc.descriptor_attention(f64(X[a:b]), f64(torch.cat(Dc[:c + 1])), p)
        assert_parity(y, ref, f"chunk {c}")
    assert cache.count == 142
    # after the last append: every frame against the whole cache
    y = attend(cache, w, d, d["X"])
    ref = odesc.descriptor_attention(f64(X), f64(torch.cat(Dc)), p)
    assert_parity(y, ref, "all frames, full cache")


def test_single_descriptor_closed_form():
    w = TINY
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    D = synth.make_descriptors(w, 1, 5)
    cache = DescriptorCache(w.d, w.H, 1)
    cache.append(D.cuda(), d["Wqkv"], d["k_gamma"], d["k_beta"])
    y = attend(cache, w, d, d["X"])
    row = (f64(D) @ f64(inp["Wqkv"])[2 * w.d:].T) @ f64(inp["Wo"]).T
    assert_parity(y, np.broadcast_to(row.reshape(1, 1, -1), y.shape), "one descriptor")


def test_descriptors_equal_tokens_is_global_bitwise():
    """A grid without patches (nothing rotated) and the tokens themselves as
    descriptors: the same projections, bounds and attention as the global
    block, so the outputs are bitwise equal."""
    w = configs.custom("desc_patchless", S=40, grid_h=0, grid_w=0, d=256, H=4, cid=64)
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    blk = api.Block("global", d["X"], w.H, 0, 0)
    yg = blk(*[d[k] for k in ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")])
    cache = DescriptorCache(w.d, w.H, w.N)
    cache.append(d["X"].reshape(-1, w.d), d["Wqkv"], d["k_gamma"], d["k_beta"])
    y = attend(cache, w, d, d["X"])
    assert torch.equal(y, yg)


def test_s100_queries_against_6400_descriptors():
    """The 100-frame token set (103,100 queries) against 64 descriptors per
    frame appended in four chunks: sampled rows against the oracle."""
    w = configs.WORKLOADS["s100"]
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    p = oracle_params(w, inp)
    Ds = [synth.make_descriptors(w, 1600, 10 + i) for i in range(4)]
    cache = DescriptorCache(w.d, w.H, 6400)
    for i, D in enumerate(Ds):
        log(f"[case] s100 descriptors: append chunk {i}")
        cache.append(D.cuda(), d["Wqkv"], d["k_gamma"], d["k_beta"])
    log("[case] s100 descriptors: attend")
    y = attend(cache, w, d, d["X"]).reshape(-1, w.d)
    rows = synth.sample_rows(w, 96).numpy()
    ref = odesc.descriptor_attention_rows(f64(inp["X"]), f64(torch.cat(Ds)), p, rows)
    assert_parity(np64(y[torch.from_numpy(rows).cuda()]), ref, "s100 x 6400")
