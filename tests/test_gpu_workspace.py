"""GPU: a call's result does not depend on what its workspace held before.

Every byte the kernels read from the workspace is written earlier in the same
call (q / k / v^T rows, the zeroed v^T columns past a frame's last row, the
scalars, the split-tail partials), so a workspace filled with NaN bit patterns
(0xFF bytes: fp16 0xFFFF, fp32 0xFFFFFFFF) gives bit for bit the output of a
zero-filled one.  Frame sets are the case to watch: their last key tile reaches
past the frame's keys into v^T columns that no token maps to, and a masked
key's zero probability times a stale NaN value would poison the row.
"""

from __future__ import annotations

import pytest
import torch

import oracle
from vggt_global_attention_amd import api, configs, synth
from helpers import assert_parity, f64, oracle_params
from gpu_common import KEYS, log, np64, require_gpu, to_dev

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
ORACLE = {"frame": oracle.frame_attention, "global": oracle.global_attention,
          "register": oracle.register_attention}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(mode, w, d, fill):
    blk = api.Block(mode, d["X"], w.H, w.grid_h, w.grid_w)
    blk.workspace.fill_(fill)
    y = blk(*[d[k] for k in KEYS])
    torch.cuda.synchronize()
    return y


# tiny (T = 81: rows 96 per frame, v^T 128), a ragged 3-frame set (T = 52:
# 64 / 64), frames of 48 tokens (48 / 64: one padding 16-group), of 64 (64 /
# 64) and of 17 (special tokens only: 32 / 64), a single frame and the
# 24-frame layer (T = 1,031: 1,040 / 1,088)
CASES = [("tiny", None), ("ragged", (3, 5, 7, 256, 4)), ("t48", (5, 1, 31, 256, 4)),
         ("t64", (4, 1, 47, 256, 4)), ("t17", (6, 0, 0, 128, 2)), ("one", (1, 26, 39, 256, 4)),
         ("s24", None)]


@pytest.mark.parametrize("mode", ["frame", "global", "register"])
@pytest.mark.parametrize("name,spec", CASES)
def test_poisoned_workspace_bitwise(name, spec, mode):
    if name == "s24" and mode != "frame":
        pytest.skip("the 24-frame layer: frame sets only (global is covered by the small sets)")
    w = W[name] if spec is None else configs.custom(name, *spec, cid=41)
    inp = synth.make_inputs(w)
    d = to_dev(inp)
    log(f"[case] poisoned workspace {name} mode={mode} S={w.S} T={w.T}")
    y0 = _run(mode, w, d, 0)
    y1 = _run(mode, w, d, 255)
    assert torch.isfinite(y1.float()).all(), f"{name}/{mode}: non-finite output"
    assert torch.equal(y0, y1), f"{name}/{mode}: output depends on stale workspace bytes"
    if w.S * w.T <= 4096:
        ref = ORACLE[mode](f64(inp["X"]), oracle_params(w, inp))
        assert_parity(np64(y1), ref, f"{name}/{mode}/poisoned")
