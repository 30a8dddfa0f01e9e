"""Torch front end of descriptor attention with a chunk-recursive key / value
cache (vggt_attn_desc_*): every image token attends to a compact set of
descriptor tokens, and chunked inference appends each chunk's descriptors to
the cache before its tokens attend ("FlashVGGT ... Compressed Descriptor
Attention", chatpaper.ai, abstract).  Buffers and streams only; the work runs
in libvggtattn.
"""

from __future__ import annotations

import torch

from . import binding as B
from .api import _stream_handle, shape_of


class DescriptorCache:
    """A key / value cache of up to `capacity` descriptors for one layer.

    The fill count lives here on the host; appends and attends are enqueued on
    the current stream without any synchronisation.
    """

    def __init__(self, d: int, H: int, capacity: int, device="cuda", ln_eps=1e-5,
                 rope_base=100.0, stream=None):
        self.d, self.H, self.capacity = int(d), int(H), int(capacity)
        self.ln_eps, self.rope_base = ln_eps, rope_base
        # only d, H and eps matter to the cache itself: a frame without patches
        self._cshape = B.make_shape(1, 17, d, H, 0, 0, rope_base, ln_eps, 0)
        n = B.vggt_attn_desc_cache_bytes(self._cshape, self.capacity)
        if n == 0:
            raise B.VggtAttnError(B.ESHAPE, "vggt_attn_desc_cache_bytes")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        self.count = 0
        self._ws = None
        self.reset(stream)

    def reset(self, stream=None):
        st = B.vggt_attn_desc_cache_init(self._cshape, self.capacity, self.buf.data_ptr(),
                                         self.buf.numel(), _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_desc_cache_init")
        self.count = 0

    def append(self, D: torch.Tensor, Wqkv, k_gamma, k_beta, stream=None):
        """Append descriptor tokens D [m, d] (bf16) with this layer's weights."""
        D = D.reshape(-1, self.d)
        if D.dtype != torch.bfloat16 or not D.is_cuda or not D.is_contiguous():
            raise ValueError("D must be a contiguous bf16 device tensor")
        m = D.shape[0]
        st = B.vggt_attn_desc_append(self._cshape, self.capacity, self.count, D.data_ptr(), m,
                                     Wqkv.data_ptr(), k_gamma.data_ptr(), k_beta.data_ptr(),
                                     self.buf.data_ptr(), self.buf.numel(), _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_desc_append")
        self.count += m

    def _args(self, X, H, grid_h, grid_w, Wqkv, Wo, q_gamma, q_beta, Y, pos_offset=0):
        shape = shape_of(X, H, grid_h, grid_w, self.rope_base, self.ln_eps, pos_offset)
        need = B.vggt_attn_workspace_bytes(B.MODE_DESCRIPTOR, shape)
        if need == 0:
            raise B.VggtAttnError(B.ESHAPE, "vggt_attn_workspace_bytes")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=X.device)
        return (shape, self.capacity, self.count, self.buf.data_ptr(), self.buf.numel(),
                X.data_ptr(), Wqkv.data_ptr(), Wo.data_ptr(), q_gamma.data_ptr(),
                q_beta.data_ptr(), Y.data_ptr(), self._ws.data_ptr(), self._ws.numel())

    def attend(self, X, grid_h, grid_w, Wqkv, Wo, q_gamma, q_beta, Y=None, stream=None,
               pos_offset=0):
        """Every token of X [S, T, d] attends to the cached descriptors."""
        if X.dtype != torch.bfloat16 or not X.is_cuda or not X.is_contiguous():
            raise ValueError("X must be a contiguous bf16 device tensor")
        if Y is None:
            Y = torch.empty_like(X)
        a = self._args(X, self.H, grid_h, grid_w, Wqkv, Wo, q_gamma, q_beta, Y, pos_offset)
        st = B.vggt_attn_desc_attend(*a, _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_desc_attend")
        return Y

    def attend_stage(self, stage, X, grid_h, grid_w, Wqkv, Wo, q_gamma, q_beta, Y, stream=None):
        a = self._args(X, self.H, grid_h, grid_w, Wqkv, Wo, q_gamma, q_beta, Y)
        st = B.vggt_attn_desc_attend_stage(stage, *a, _stream_handle(stream))
        if st != B.OK:
            raise B.VggtAttnError(st, "vggt_attn_desc_attend_stage")
        return Y
