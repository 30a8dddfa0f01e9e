"""fp64 CPU oracle of descriptor cross-attention with a chunk-recursive cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the GPU library; it
shares no code with the HIP path.  The projections (QKV, per-head LayerNorm,
2D RoPE) are those of `vggt_oracle`.

Source: "FlashVGGT: Efficient and Scalable Visual Geometry Transformers with
Compressed Descriptor Attention" (chatpaper.ai, abstract).  Instead of dense
global attention over all tokens, each frame's spatial information is
compressed into a small set of descriptor tokens, and the global step becomes
cross-attention from the full set of image tokens to the descriptor set.  For
long sequences, inference runs chunk by chunk and reuses the cached
descriptors of earlier chunks.

Readings (the abstract leaves them open):
* The compression itself is not described (it is presumably learned): the
  descriptor tokens are an input, token states of width d like X.
* Queries: every image token, projected, LayerNorm-ed and rotated exactly as
  in the global block.  Keys / values: the descriptor tokens through the same
  layer's Wqkv (K and V rows) and key LayerNorm.  Descriptors have no place on
  the patch grid, so they are not rotated (like camera and register tokens).
* softmax(q k^T / sqrt(Dh)) v per head over all cached descriptors, heads
  concatenated, times Wo^T.  No mask: every query sees every descriptor.
* Chunk recursion: chunk c's descriptors join the cache, then chunk c's
  tokens attend to everything cached so far (its own and all earlier chunks'
  descriptors, never later ones).
"""

from __future__ import annotations

import numpy as np

from .vggt_oracle import OracleParams, _attend, _project, default_threads


def descriptor_kv(D: np.ndarray, p: OracleParams):
    """Keys (normalised, not rotated) and values of descriptor tokens D [M, d]."""
    D = np.asarray(D, dtype=np.float64).reshape(-1, p.d)
    t = np.zeros(len(D), dtype=np.int64)      # token index 0: no grid position
    kv = _project(D, t, p, want=("k", "v"))
    return kv["k"], kv["v"]


def descriptor_attention(X: np.ndarray, D: np.ndarray, p: OracleParams,
                         threads: int | None = None) -> np.ndarray:
    """Every token of X [S, T, d] attends to the descriptor tokens D [M, d]."""
    threads = threads or default_threads()
    S, T, d = X.shape
    if T != p.T or d != p.d:
        raise ValueError("shape mismatch")
    if len(D) < 1:
        raise ValueError("at least one descriptor")
    Xf = np.asarray(X, dtype=np.float64).reshape(S * T, d)
    t = np.tile(np.arange(T), S)
    q = _project(Xf, t, p, want=("q",))["q"]
    k, v = descriptor_kv(D, p)
    O = _attend(q, k, v, threads)
    return (O @ p.Wo.T).reshape(S, T, d)


def descriptor_attention_rows(X: np.ndarray, D: np.ndarray, p: OracleParams, rows,
                              threads: int | None = None) -> np.ndarray:
    """Rows (flat token indices s*T + t) of descriptor_attention."""
    threads = threads or default_threads()
    S, T, d = X.shape
    rows = np.asarray(rows, dtype=np.int64)
    Xf = np.asarray(X, dtype=np.float64).reshape(S * T, d)
    q = _project(Xf[rows], rows % T, p, want=("q",))["q"]
    k, v = descriptor_kv(D, p)
    return _attend(q, k, v, threads) @ p.Wo.T


def chunk_recursive(X_chunks: list, D_chunks: list, p: OracleParams,
                    threads: int | None = None) -> list:
    """Online inference over chunks: chunk c's descriptors are appended to the
    cache, then chunk c's tokens attend to the whole cache.  Returns the list
    of per-chunk outputs."""
    cache = []
    out = []
    for Xc, Dc in zip(X_chunks, D_chunks):
        cache.append(np.asarray(Dc, dtype=np.float64).reshape(-1, p.d))
        out.append(descriptor_attention(Xc, np.concatenate(cache), p, threads))
    return out
