"""Torch-tensor front end of libvggtattn (device memory and streams only).

torch supplies the device buffers and the current HIP stream; the ctypes call
does all the work.  Nothing here computes any part of the attention block.
"""

from __future__ import annotations

import torch

from . import binding as B

_ENTRY = {"frame": "vggt_attn_frame", "global": "vggt_attn_global",
          "register": "vggt_attn_global_register", "subsampled": "vggt_attn_global_subsampled",
          "merged": "vggt_attn_global_merged"}


def shape_of(X: torch.Tensor, H: int, grid_h: int, grid_w: int, rope_base=100.0,
             ln_eps=1e-5, pos_offset=0) -> B.vggt_attn_shape:
    S, T, d = X.shape
    return B.make_shape(S, T, d, H, grid_h, grid_w, rope_base, ln_eps, pos_offset)


def workspace_bytes(mode: str, shape: B.vggt_attn_shape) -> int:
    n = B.vggt_attn_workspace_bytes(B.MODES[mode], shape)
    if n == 0:
        raise B.VggtAttnError(B.ESHAPE, "vggt_attn_workspace_bytes")
    return n


def alloc_workspace(mode: str, shape: B.vggt_attn_shape, device) -> torch.Tensor:
    return torch.empty(workspace_bytes(mode, shape), dtype=torch.uint8, device=device)


def _check_tensors(X, Wqkv, Wo, gb):
    for name, t, dt in (("X", X, torch.bfloat16), ("Wqkv", Wqkv, torch.bfloat16),
                        ("Wo", Wo, torch.bfloat16)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    for t in gb:
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("gamma/beta must be contiguous float32 device tensors")


def _stream_handle(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Block:
    """One attention block configuration with its workspace, reusable across calls."""

    def __init__(self, mode: str, X: torch.Tensor, H: int, grid_h: int, grid_w: int,
                 rope_base=100.0, ln_eps=1e-5, pos_offset=0, workspace=None, sub=(1, 1),
                 merge=(2, 1, 1, 0), operands="fp16"):
        if mode not in _ENTRY:
            raise ValueError(f"unknown mode {mode!r}")
        if operands not in ("fp16", "bf16"):
            raise ValueError(f"unknown attention operand type {operands!r}")
        if operands == "bf16" and mode not in ("frame", "global", "register"):
            raise ValueError("bf16 attention operands serve the frame, global and register modes")
        self.mode = mode
        # attention operands (q, k, v, P, O, Wo copy): fp16, or the bf16 variant
        self.bf16 = operands == "bf16"
        self.sub = (int(sub[0]), int(sub[1]))  # subsampled mode: (sub_h, sub_w) windows
        # merged mode: (frames per block, window rows, window columns, merges per block)
        self.merge = tuple(int(x) for x in merge)
        self.shape = shape_of(X, H, grid_h, grid_w, rope_base, ln_eps, pos_offset)
        need = workspace_bytes(mode, self.shape)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        self.workspace = workspace

    def _args(self, X, Wqkv, Wo, qg, qb, kg, kb, Y):
        _check_tensors(X, Wqkv, Wo, (qg, qb, kg, kb))
        return (self.shape, X.data_ptr(), Wqkv.data_ptr(), Wo.data_ptr(), qg.data_ptr(),
                qb.data_ptr(), kg.data_ptr(), kb.data_ptr(), Y.data_ptr(),
                self.workspace.data_ptr(), self.workspace.numel())

    def __call__(self, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y=None, stream=None):
        if Y is None:
            Y = torch.empty_like(X)
        args = self._args(X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y)
        if self.mode == "subsampled":
            st = B.vggt_attn_global_subsampled(args[0], *self.sub, *args[1:],
                                               _stream_handle(stream))
        elif self.mode == "merged":
            st = B.vggt_attn_global_merged(args[0], *self.merge, *args[1:],
                                           _stream_handle(stream))
        elif self.bf16:
            st = B.vggt_attn_bf16ops(B.MODES[self.mode], B.STAGE_ALL, *args,
                                     _stream_handle(stream))
        else:
            st = getattr(B, _ENTRY[self.mode])(*args, _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, _ENTRY[self.mode])
        return Y

    def stage(self, stage: int, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y, stream=None):
        args = self._args(X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y)
        if self.mode == "subsampled":
            st = B.vggt_attn_subsampled_stage(stage, args[0], *self.sub, *args[1:],
                                              _stream_handle(stream))
        elif self.mode == "merged":
            st = B.vggt_attn_merged_stage(stage, args[0], *self.merge, *args[1:],
                                          _stream_handle(stream))
        elif self.bf16:
            st = B.vggt_attn_bf16ops(B.MODES[self.mode], stage, *args, _stream_handle(stream))
        else:
            st = B.vggt_attn_stage(B.MODES[self.mode], stage, *args, _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_stage")
        return Y


class RowsBlock:
    """Rows [row_begin, row_begin + row_count) of the global block (one GPU's
    share of a query-row split), with its workspace."""

    def __init__(self, X: torch.Tensor, H: int, grid_h: int, grid_w: int, row_begin: int,
                 row_count: int, rope_base=100.0, ln_eps=1e-5, pos_offset=0, workspace=None):
        self.inner = Block("global", X, H, grid_h, grid_w, rope_base, ln_eps, pos_offset,
                           workspace)
        self.row_begin, self.row_count = int(row_begin), int(row_count)

    def _args(self, X, Wqkv, Wo, qg, qb, kg, kb, Y):
        return self.inner._args(X, Wqkv, Wo, qg, qb, kg, kb, Y)

    def __call__(self, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y=None, stream=None):
        if Y is None:
            Y = torch.empty((self.row_count, X.shape[-1]), dtype=X.dtype, device=X.device)
        a = self._args(X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y)
        st = B.vggt_attn_global_rows(a[0], self.row_begin, self.row_count, *a[1:],
                                     _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_global_rows")
        return Y

    def stage(self, stage: int, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y, stream=None):
        a = self._args(X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y)
        st = B.vggt_attn_global_rows_stage(stage, a[0], self.row_begin, self.row_count, *a[1:],
                                           _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_global_rows_stage")
        return Y


def attention(mode: str, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, H: int, grid_h: int,
              grid_w: int, Y=None, stream=None, sub=(1, 1), merge=(2, 1, 1, 0), **shape_kw):
    """One call of the block in `mode` ('frame', 'global', 'register', 'subsampled' or
    'merged'; `sub` = (sub_h, sub_w) windows of the subsampled mode, `merge` = (frames,
    window rows, window columns, merges per block) of the merged mode)."""
    blk = Block(mode, X, H, grid_h, grid_w, sub=sub, merge=merge, **shape_kw)
    return blk(X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y=Y, stream=stream)
