"""HIP graph capture of library calls.

The library only launches kernels on the caller's stream. It makes no memset,
copy or allocation, so a call can be captured into a HIP graph
(torch.cuda.CUDAGraph) and replayed.

Each graph is replayed several times, with the program's own eager work and
synchronisations in between (the outputs are cleared first). Every replay
must equal the eager result bit for bit.
"""

from __future__ import annotations

import pytest
import torch

from vggt_global_attention_amd import api, configs, synth
from vggt_global_attention_amd import schedule as S
from gpu_common import log, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def capture(fn):
    """fn() captured on a side stream into a graph (after one eager warm-up on
    that stream, which also fills the library's per-device caches)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outs, refs, label, n=3):
    for i in range(n):
        for o in outs:
            o.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"{label}: replay {i}"


def test_schedule_graph_replay():
    """The 24-layer forward of three frames (48 blocks, 48 residual updates,
    the four kept states) as one graph."""
    w = configs.custom("graph_sched", S=3, grid_h=4, grid_w=5, d=256, H=4, cid=71)
    blocks = [{k: v.cuda().contiguous() for k, v in b.items()}
              for b in synth.make_block_weights(w, 48, 0.25)]
    X = synth.make_inputs(w)["X"].cuda()
    sch = S.Schedule(X, w.H, w.grid_h, w.grid_w, blocks)
    state = torch.empty_like(X)
    caches = sch.alloc_caches(X)
    sch(X, state=state, caches=caches)
    torch.cuda.synchronize()
    ref = (state.clone(), caches.clone())
    log("[case] graph of the 24-layer schedule, S=3")
    g = capture(lambda: sch(X, state=state, caches=caches))
    replay_and_check(g, (state, caches), ref, "schedule")


@pytest.mark.parametrize("mode,ops", [("global", "fp16"), ("frame", "fp16"), ("register", "fp16"),
                                     ("subsampled", "fp16"), ("merged", "fp16"),
                                     ("global", "bf16")])
def test_block_graph_replay(mode, ops):
    """One block call of 24 frames. The global block runs a split tail (key
    ranges and the merge kernel), captured like any other launch; the merged
    block's merge and unmerge kernels and the bf16-operand variant too."""
    w = configs.WORKLOADS["s24"]
    d = to_dev(synth.make_inputs(w))
    sub = (3, 3) if mode == "subsampled" else (1, 1)
    blk = api.Block(mode, d["X"], w.H, w.grid_h, w.grid_w, sub=sub, merge=(4, 2, 3, 12),
                    operands=ops)
    args = [d[k] for k in ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")]
    Y = torch.empty_like(d["X"])
    blk(*args, Y=Y)
    torch.cuda.synchronize()
    ref = Y.clone()
    log(f"[case] graph of one {mode} block ({ops} operands), s24")
    g = capture(lambda: blk(*args, Y=Y))
    replay_and_check(g, (Y,), (ref,), f"{mode}/{ops}")
