"""fp64 CPU oracle of AVGGT subsampled global attention (SGA).

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's CPU
baseline leg, never by the GPU library, and it shares no code with the HIP
path.  Float64 NumPy throughout; the q, k, v projections (QKV, per-head
LayerNorm, 2D RoPE) are those of `vggt_oracle`.

Source: "AVGGT: Rethinking Global Attention for Accelerating VGGT", summary on
gist.science, technical summary section 2B ("Subsampling van Globale
Attention"), three points, taken in that order:

1. Grid subsampling of keys and values.  Every query of the global set is
   kept, but only a sparse, uniform subset of the patch tokens serves as keys
   and values: one token per s_h x s_w window of the patch grid.
   Readings (the page leaves them open): the kept token of a window is its
   top-left cell, i.e. patch (r, c) is kept iff r % s_h == 0 and c % s_w == 0
   (windows cut by the grid edge still keep their top-left cell); the camera
   and register tokens are not patch tokens and are always kept.
2. Diagonal kept.  Each token still attends to its own key and value.
3. Mean fill.  All discarded columns are stood in for by one mean key/value
   pair, the mean of the discarded keys and of the discarded values.  Reading:
   "fill" is taken literally -- every column of the full attention row that
   is neither kept nor the row's own diagonal is replaced by that mean pair,
   so the pair enters the softmax with multiplicity n_i = |D| - [i in D]
   (D = discarded tokens).  With s_h = s_w = 1 nothing is discarded and the
   result is exact global attention; if all discarded keys and values were
   equal, it would also be exact.  The means are taken over the normalised,
   rotated keys (the keys as attention sees them) and the raw values, per
   head.

Everything after attention (heads concatenated, times Wo^T) is as in the
global block.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .vggt_oracle import (N_SPECIAL, OracleParams, _NullCtx, _check, _project,
                          default_threads, threadpool_limits)


def kept_tokens(S: int, grid_h: int, grid_w: int, sub_h: int, sub_w: int) -> np.ndarray:
    """Boolean [S*T]: token is a key/value of the subsampled set (point 1)."""
    if sub_h < 1 or sub_w < 1:
        raise ValueError("sub_h and sub_w must be >= 1")
    T = N_SPECIAL + grid_h * grid_w
    t = np.arange(T)
    p = t - N_SPECIAL
    r, c = p // max(grid_w, 1), p % max(grid_w, 1)
    frame = (t < N_SPECIAL) | ((r % sub_h == 0) & (c % sub_w == 0))
    return np.tile(frame, S)


def diagonal_columns(kept_rows: np.ndarray) -> np.ndarray:
    """Point 2: rows whose own key/value is an extra column (not already kept)."""
    return ~kept_rows


def mean_multiplicity(n_discarded: int, diag_on: np.ndarray) -> np.ndarray:
    """Point 3: how many columns of the row the mean pair fills."""
    return n_discarded - diag_on.astype(np.int64)


def sga_core(q: np.ndarray, k: np.ndarray, v: np.ndarray, kept: np.ndarray, rows=None,
             threads: int | None = None, chunk: int = 256) -> np.ndarray:
    """SGA on projected tensors: k, v [N, H, Dh], kept bool [N]; q [len(rows), H, Dh]
    holds the queries of the tokens `rows` (default: all N tokens, q [N, H, Dh]).

    Returns O [len(rows), H*Dh].
    Per query i and head: logits q_i.k_j / sqrt(Dh) over the kept columns j,
    the diagonal column (only if i is not kept: otherwise it is already among
    the kept ones), and the mean column with logit q_i.kbar / sqrt(Dh) and
    multiplicity n_i; softmax over all of them; O_i = sum_j P_ij v_j + n_i P_mean vbar.
    """
    threads = threads or default_threads()
    N, H, Dh = k.shape
    kept = np.asarray(kept, dtype=bool)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    if q.shape != (len(rows), H, Dh):
        raise ValueError(f"q {q.shape} does not match {len(rows)} rows of k {k.shape}")
    K_idx = np.nonzero(kept)[0]
    D_idx = np.nonzero(~kept)[0]
    nD = len(D_idx)
    scale = 1.0 / math.sqrt(Dh)
    O = np.empty((len(rows), H, Dh), dtype=np.float64)
    # point 3: one mean pair per head over the discarded tokens
    if nD > 0:
        kbar = k[D_idx].mean(axis=0)   # [H, Dh]
        vbar = v[D_idx].mean(axis=0)
    else:
        kbar = np.zeros((H, Dh))
        vbar = np.zeros((H, Dh))
    kK = [np.ascontiguousarray(k[K_idx, h]) for h in range(H)]
    vK = [np.ascontiguousarray(v[K_idx, h]) for h in range(H)]

    def job(h, lo):
        hi = min(len(rows), lo + chunk)
        ri = rows[lo:hi]
        qh = q[lo:hi, h]                                # [m, Dh]
        a_kept = (qh @ kK[h].T) * scale                 # [m, |K|]   point 1
        diag_on = diagonal_columns(kept[ri])            # point 2
        a_diag = np.einsum("md,md->m", qh, k[ri, h]) * scale
        n_i = mean_multiplicity(nD, diag_on)            # point 3
        a_mean = (qh @ kbar[h]) * scale
        # one softmax over [kept | diagonal | mean x n_i]
        with np.errstate(divide="ignore"):
            log_n = np.where(n_i > 0, np.log(np.maximum(n_i, 1)), -np.inf)
        cols = np.concatenate(
            [a_kept, np.where(diag_on, a_diag, -np.inf)[:, None], (a_mean + log_n)[:, None]], axis=1)
        cols -= cols.max(axis=1, keepdims=True)
        e = np.exp(cols)
        P = e / e.sum(axis=1, keepdims=True)
        O[lo:hi, h] = (P[:, :-2] @ vK[h] + P[:, -2:-1] * v[ri, h] + P[:, -1:] * vbar[h])

    jobs = [(h, lo) for h in range(H) for lo in range(0, len(rows), chunk)]
    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            job(*j)
    else:
        limiter = threadpool_limits(limits=1) if threadpool_limits else _NullCtx()
        with limiter, ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda j: job(*j), jobs))
    return O.reshape(len(rows), H * Dh)


def sga_attention(X: np.ndarray, p: OracleParams, sub_h: int, sub_w: int,
                  threads: int | None = None) -> np.ndarray:
    """Global block with SGA: Y [S, T, d] for every token."""
    S, T, d = _check(X, p)
    Xf = X.reshape(S * T, d).astype(np.float64)
    t = np.tile(np.arange(T), S)
    qkv = _project(Xf, t, p)
    kept = kept_tokens(S, p.grid_h, p.grid_w, sub_h, sub_w)
    O = sga_core(qkv["q"], qkv["k"], qkv["v"], kept, threads=threads)
    return (O @ p.Wo.T).reshape(S, T, d)


def sga_attention_rows(X: np.ndarray, p: OracleParams, sub_h: int, sub_w: int, rows,
                       threads: int | None = None) -> np.ndarray:
    """Y at the flat rows `rows` (row = s*T + t); keys, values and means span the set."""
    S, T, d = _check(X, p)
    rows = np.asarray(rows, dtype=np.int64)
    Xf = X.reshape(S * T, d)
    t_all = np.tile(np.arange(T), S)
    kv = _project(Xf.astype(np.float64), t_all, p, want=("k", "v"))
    q = _project(Xf[rows].astype(np.float64), t_all[rows], p, want=("q",))["q"]
    kept = kept_tokens(S, p.grid_h, p.grid_w, sub_h, sub_w)
    O = sga_core(q, kv["k"], kv["v"], kept, rows=rows, threads=threads)
    return O @ p.Wo.T
