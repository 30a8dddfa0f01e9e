"""Torch front end of the layer-schedule entry point (vggt_attn_schedule_run).

The schedule itself -- which block runs in which mode, the residual updates
with LayerScale, the kept states -- runs inside libvggtattn as one call; this
module fills the C structs and owns the device buffers.

Defaults follow "VGGT-Omega Aggregator explainer" (ksqn.cn): 24 layers,
register-mode inter-frame blocks at layers [2, 6, 9, 14, 20] (0-based), states
kept at layers [4, 11, 17, 23] (sections 三 and 四).  `early_frame` and `sub`
are AVGGT's conversions (AVGGT summary, technical summary 2B).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import binding as B
from .api import _stream_handle, shape_of

REGISTER_LAYERS = (2, 6, 9, 14, 20)
CACHED_LAYERS = (4, 11, 17, 23)
N_LAYERS = 24


def layer_mask(layers) -> int:
    m = 0
    for l in layers:
        m |= 1 << int(l)
    return m


@dataclass
class ScheduleSpec:
    n_layers: int = N_LAYERS
    register_layers: tuple = REGISTER_LAYERS
    cached_layers: tuple = CACHED_LAYERS
    early_frame: int = 0
    sub: tuple = field(default=(1, 1))
    # HTTM merging in the global inter-frame blocks: (frames per block, window
    # rows, window columns, merges per block), or None
    merge: tuple = None

    def c_struct(self) -> B.vggt_attn_schedule:
        m = tuple(int(x) for x in self.merge) if self.merge else (0, 0, 0, 0)
        return B.vggt_attn_schedule(self.n_layers, self.early_frame,
                                    layer_mask(self.register_layers),
                                    layer_mask(self.cached_layers), int(self.sub[0]),
                                    int(self.sub[1]), *m)

    def inter_mode(self, l: int) -> str:
        """Mode of layer l's inter-frame block (host bookkeeping, e.g. FLOP counts)."""
        if l in self.register_layers:
            return "register"
        if l < self.early_frame:
            return "frame"
        if self.merge:
            return "merged"
        return "subsampled" if tuple(self.sub) != (1, 1) else "global"


def _check_block(w: dict, d: int):
    for name in ("Wqkv", "Wo"):
        t = w[name]
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 device tensor")
    for name in ("q_gamma", "q_beta", "k_gamma", "k_beta", "layer_scale"):
        t = w[name]
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if w["layer_scale"].numel() != d:
        raise ValueError("layer_scale must hold d values")


class Schedule:
    """A layer schedule bound to a shape, its block weights and workspace.

    `blocks` holds 2 * n_layers dicts of device tensors (keys Wqkv, Wo,
    q_gamma, q_beta, k_gamma, k_beta, layer_scale): entry 2l is layer l's frame
    block, 2l + 1 its inter-frame block.
    """

    def __init__(self, X: torch.Tensor, H: int, grid_h: int, grid_w: int, blocks: list,
                 spec: ScheduleSpec | None = None, workspace=None, **shape_kw):
        self.spec = spec or ScheduleSpec()
        if len(blocks) != 2 * self.spec.n_layers:
            raise ValueError(f"need {2 * self.spec.n_layers} blocks, got {len(blocks)}")
        self.shape = shape_of(X, H, grid_h, grid_w, **shape_kw)
        self.sched = self.spec.c_struct()
        need = B.vggt_attn_schedule_workspace_bytes(self.shape, self.sched)
        if need == 0:
            raise B.VggtAttnError(B.ESHAPE, "vggt_attn_schedule_workspace_bytes")
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        self.workspace = workspace
        d = X.shape[-1]
        for w in blocks:
            _check_block(w, d)
        self._blocks = blocks  # keeps the tensors alive
        arr = (B.vggt_attn_block_weights * len(blocks))()
        for i, w in enumerate(blocks):
            arr[i] = B.vggt_attn_block_weights(
                w["Wqkv"].data_ptr(), w["Wo"].data_ptr(), w["q_gamma"].data_ptr(),
                w["q_beta"].data_ptr(), w["k_gamma"].data_ptr(), w["k_beta"].data_ptr(),
                w["layer_scale"].data_ptr())
        self._arr = arr

    @property
    def n_cached(self) -> int:
        return len(self.spec.cached_layers)

    def alloc_caches(self, X: torch.Tensor) -> torch.Tensor:
        S, T, d = X.shape
        return torch.empty((self.n_cached, S, T, 2 * d), dtype=X.dtype, device=X.device)

    def __call__(self, X: torch.Tensor, state=None, caches=None, keep=True, stream=None):
        """Run the schedule on X; returns (state, caches).  `state` may be X
        (in place).  keep=False skips the kept states (caches is then None)."""
        if X.dtype != torch.bfloat16 or not X.is_cuda or not X.is_contiguous():
            raise ValueError("X must be a contiguous bf16 device tensor")
        if state is None:
            state = torch.empty_like(X)
        if keep and self.n_cached and caches is None:
            caches = self.alloc_caches(X)
        if not keep:
            caches = None
        st = B.vggt_attn_schedule_run(self.shape, self.sched, self._arr, X.data_ptr(),
                                      state.data_ptr(), caches.data_ptr() if caches is not None
                                      else None, self.workspace.data_ptr(),
                                      self.workspace.numel(), _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_schedule_run")
        return state, caches


def residual(X, Y, gamma, Z=None, period=1, active=1, C=None, c_stride=None, stream=None):
    """Z = X + gamma * Y on rows r with r % period < active (Z = X elsewhere)."""
    d = X.shape[-1]
    rows = X.numel() // d
    if Z is None:
        Z = torch.empty_like(X)
    st = B.vggt_attn_residual(X.data_ptr(), Y.data_ptr(), Z.data_ptr(), rows, d,
                              gamma.data_ptr(), period, active,
                              C.data_ptr() if C is not None else None,
                              c_stride if c_stride is not None else d, _stream_handle(stream))
    if st != B.OK:
        raise B.VggtAttnError(st, "vggt_attn_residual")
    return Z
