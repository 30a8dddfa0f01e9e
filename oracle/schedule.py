"""fp64 CPU oracle of the Aggregator's attention-only layer schedule.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the GPU library; it
shares no code with the HIP path.  The blocks are those of `vggt_oracle` and
`avggt_sga` and `httm`; this module only composes them.

Sources and readings:

* "VGGT-Omega Aggregator explainer" (ksqn.cn), section 三: the Aggregator is 24
  layers deep; every layer runs a frame block and then an inter-frame block.
  The inter-frame block is in register mode at the five layer indices
  [2, 6, 9, 14, 20] and global elsewhere.  Readings: the indices count layers
  from 0; "register mode at those layers" (not "global at those layers").
  In register mode the patch tokens keep to their own frame, read as: the
  inter-frame block leaves patch rows unchanged, only the 17 special tokens
  of every frame are updated.
* Same page, section 三: attention layers use LayerScale (initialised to
  1e-5).  Read as the usual residual branch: x <- x + gamma * block(x) with
  one gamma per channel and per block; the trained values are not on the
  page, so they are inputs here.
* Same page, section 四: the states of layers 4, 11, 17 and 23 are kept, the
  frame block's output and the inter-frame block's output concatenated along
  channels (2 x 1024 features).  Read as: the token state after the frame
  block's residual update, then the state after the inter-frame block's.
* AVGGT summary (gist.science), technical summary 2B, step 1: early global
  layers become frame attention (same weights, attention inside each frame);
  step 2: the remaining global layers use subsampled global attention.  How
  many layers count as "early" is not given: it is a parameter.
* "HTTM" article (10100.com), section 02: token merging is designed for
  VGGT's global attention layers; read as: with merging on, every global
  inter-frame block (not register, not early frame) runs with it, with one
  parameter set for all (`httm`).
* Storage: the token state and every block output are bf16, the library's
  input/output type.  The oracle computes each block and each residual update
  in float64 from the exact bf16 values and rounds the result once to the
  nearest bf16 (ties to even), as the state's storage format demands.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .avggt_sga import sga_attention
from .httm import HttmParams, httm_attention
from .vggt_oracle import (N_SPECIAL, OracleParams, frame_attention, global_attention,
                          register_attention)

REGISTER_LAYERS = (2, 6, 9, 14, 20)   # section 三
CACHED_LAYERS = (4, 11, 17, 23)       # section 四
N_LAYERS = 24                         # section 三


@dataclass
class Spec:
    n_layers: int = N_LAYERS
    register_layers: tuple = REGISTER_LAYERS
    cached_layers: tuple = CACHED_LAYERS
    early_frame: int = 0          # AVGGT step 1: layers below this run frame attention
    sub: tuple = field(default=(1, 1))  # AVGGT step 2: windows of the remaining global layers
    merge: tuple = None           # HTTM: (frames, win_h, win_w, r) of the remaining global layers

    def inter_mode(self, l: int) -> str:
        if l in self.register_layers:
            return "register"
        if l < self.early_frame:
            return "frame"
        if self.merge:
            return "merged"
        if tuple(self.sub) != (1, 1):
            return "subsampled"
        return "global"

    def params(self, mode: str):
        """The extra parameters of an inter-frame block in `mode`."""
        return tuple(self.merge) if mode == "merged" else tuple(self.sub)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of float64 x.

    Written from the format: x = m * 2**e with 0.5 <= |m| < 1, so m * 2**8 has
    8 integer bits; np.round rounds halves to even.  Normal range only (the
    states here stay far from bf16's underflow and overflow).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def inter_block(x: np.ndarray, p: OracleParams, mode: str, sub, threads=None) -> np.ndarray:
    """One inter-frame block; `sub` holds the mode's parameters (the windows
    of subsampled mode, the four merge parameters of merged mode)."""
    if mode == "frame":
        return frame_attention(x, p, threads)
    if mode == "global":
        return global_attention(x, p, threads)
    if mode == "register":
        return register_attention(x, p, threads)
    if mode == "subsampled":
        return sga_attention(x, p, sub[0], sub[1], threads=threads)
    if mode == "merged":
        return httm_attention(x, p, HttmParams(*sub), threads=threads)
    raise ValueError(mode)


def run_schedule(X: np.ndarray, blocks: list, layer_scales: list, spec: Spec, threads=None,
                 trace: bool = False, perturb=None):
    """The attention-only forward over `spec.n_layers` layers.

    X: [S, T, d] (exact bf16 values); blocks[2l] / blocks[2l+1]: OracleParams
    of layer l's frame / inter-frame block; layer_scales: matching [d] vectors.
    Returns (state, caches) -- caches [n_cached, S, T, 2d] in increasing layer
    order -- and, with trace=True, also the list of (a_l, x_l) states of every
    layer (a_l after the frame block, x_l after the inter-frame block).
    perturb(y, block_index) -> y, when given, replaces each block's exact
    output before its bf16 rounding (a model of a computation with per-block
    errors, for deriving how far such errors carry through the layers).
    """
    keep = (lambda y, b: y) if perturb is None else perturb
    x = np.asarray(X, dtype=np.float64)
    T = x.shape[1]
    special = (np.arange(T) < N_SPECIAL)[None, :, None]
    caches, states = [], []
    for l in range(spec.n_layers):
        y = round_bf16(keep(frame_attention(x, blocks[2 * l], threads), 2 * l))
        a = round_bf16(x + layer_scales[2 * l] * y)
        mode = spec.inter_mode(l)
        y = round_bf16(keep(inter_block(a, blocks[2 * l + 1], mode, spec.params(mode), threads),
                            2 * l + 1))
        upd = round_bf16(a + layer_scales[2 * l + 1] * y)
        x = np.where(special, upd, a) if mode == "register" else upd
        if l in spec.cached_layers:
            caches.append(np.concatenate([a, x], axis=-1))
        if trace:
            states.append((a, x))
    caches = np.stack(caches) if caches else np.zeros((0,) + x.shape[:2] + (2 * x.shape[2],))
    return (x, caches, states) if trace else (x, caches)
