"""GPU check of vggt_attn_block_noalloc, the block call whose workspace is the
library's static device scratch (for callers that cannot allocate).

Through the C ABI, against the block call of the same mode with a workspace
of its own: two calls in a row on the shared scratch, the second with a
smaller input, each bit for bit the existing entry point's output (the same
kernels on the same plan); then a call beyond the scratch, which must be
rejected with nothing written.
"""

from __future__ import annotations

import pytest
import torch

from vggt_global_attention_amd import api, configs, synth
from vggt_global_attention_amd import binding as B
from gpu_common import log, require_gpu, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")
ENTRY = {"frame": B.vggt_attn_frame, "global": B.vggt_attn_global,
         "register": B.vggt_attn_global_register}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def with_workspace(mode, w, d):
    """The existing entry point of `mode`, with a workspace of its own."""
    shape = api.shape_of(d["X"], w.H, w.grid_h, w.grid_w)
    ws = api.alloc_workspace(mode, shape, d["X"].device)
    Y = torch.full_like(d["X"], float("nan"))
    st = ENTRY[mode](shape, *[d[k].data_ptr() for k in KEYS], Y.data_ptr(), ws.data_ptr(),
                     ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == B.OK, st
    return Y


def noalloc(mode, w, d):
    shape = api.shape_of(d["X"], w.H, w.grid_h, w.grid_w)
    Y = torch.full_like(d["X"], float("nan"))
    st = B.vggt_attn_block_noalloc(B.MODES[mode], shape, *[d[k].data_ptr() for k in KEYS],
                                   Y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == B.OK, (mode, st, B.status_str(st))
    return Y


# (larger, smaller) pairs per mode, each within the static scratch
PAIRS = {
    "global": (configs.custom("na_g1", 6, 26, 39, 1024, 16, cid=81),
               configs.custom("na_g2", 2, 7, 11, 256, 4, cid=82)),
    "frame": (configs.custom("na_f1", 12, 26, 39, 1024, 16, cid=83),
              configs.custom("na_f2", 3, 5, 7, 128, 2, cid=84)),
    "register": (configs.custom("na_r1", 500, 26, 39, 1024, 16, cid=85),
                 configs.custom("na_r2", 40, 26, 39, 1024, 16, cid=86)),
}


@pytest.mark.parametrize("mode", ["global", "frame", "register"])
def test_noalloc_matches_the_block_call(mode):
    for w in PAIRS[mode]:
        log(f"[case] noalloc {mode} S={w.S} T={w.T} d={w.d} H={w.H}")
        d = to_dev(synth.make_inputs(w))
        y = noalloc(mode, w, d)
        torch.cuda.synchronize()
        ref = with_workspace(mode, w, d)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (mode, w.name)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    w = configs.custom("na_big", 10, 26, 39, 1024, 16, cid=87)
    log(f"[case] noalloc beyond the scratch: global S={w.S}")
    d = to_dev(synth.make_inputs(w))
    shape = api.shape_of(d["X"], w.H, w.grid_h, w.grid_w)
    assert B.vggt_attn_workspace_bytes(B.MODE_GLOBAL, shape) > B.STATIC_SCRATCH_BYTES
    Y = torch.full_like(d["X"], 7.0)
    st = B.vggt_attn_block_noalloc(B.MODE_GLOBAL, shape, *[d[k].data_ptr() for k in KEYS],
                                   Y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == B.ESCRATCH
    assert bool((Y == 7.0).all())
