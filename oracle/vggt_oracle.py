"""fp64 CPU oracle of the VGGT Aggregator attention block (frame / global / register).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the GPU library.  It shares no code with
the HIP path.  Everything is evaluated in float64 with NumPy; the inputs are the
exact float64 values of the bf16 / fp32 tensors the GPU receives.

What it computes (the plain definition, no tiling, no online softmax):

* Token recipe -- "VGGT-Omega Aggregator explainer" (ksqn.cn), section 二: each
  frame is [1 camera token][16 register tokens][patch tokens], the patches
  coming from 16x16 pixel cells of the image, so T = 17 + grid_h * grid_w.
  Patches are taken in row-major order of the grid (a reading: the page does
  not spell the order out).
* Frame block -- same page, section 三: self-attention restricted to the tokens
  of one frame, with a two-dimensional rotary position encoding.
* Inter-frame block, global mode -- same page, section 三: the tokens of all
  frames are laid end to end as one long sequence and attend to each other
  without restriction.  HTTM article (10100.com), section 02, and the AVGGT
  summary (gist.science), technical summary 1-2, make the same point: this is
  the quadratic, dominant cost.
* Inter-frame block, register mode -- same page, section 三: only the camera
  token and the 16 register tokens of every frame (17 per frame) take part in
  cross-frame attention; patch tokens stay on their own per-frame path, so the
  block leaves them unchanged here.
* Q/K normalisation -- same page, section 三 ("use_qk_norm" is on).  Read as a
  LayerNorm over the Dh features of every (token, head), biased variance,
  followed by a per-head affine gamma/beta.
* 2D RoPE -- same page, section 三 (frame block), and the HTTM article
  ("HTTM: Head-wise Temporal Token Merging for Faster VGGT", 10100.com),
  section 04, RoPE-effect paragraph around figure 3: the rotary code is
  applied in every attention layer and identically in every frame, nothing
  marks the frame index.  Read as: the first Dh/2 features are rotated by the
  patch's grid row, the last Dh/2 by its grid column; inside each half, feature
  i pairs with feature i + Dh/4 (rotate-half) and turns by pos * theta_i with
  theta_i = base ** (-i / (Dh/4)).  Special tokens are not rotated.  Applied to
  the normalised q and k, never to v.
* Attention -- softmax(q k^T / sqrt(Dh)) v per head, no mask inside a set; heads
  are concatenated head-major and multiplied by Wo^T.  No bias, no residual.

Wqkv rows are [Q heads 0..H-1 ; K heads ; V heads], Dh rows per head.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

try:  # keep BLAS single-threaded inside the worker pool (no oversubscription)
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover - threadpoolctl is optional
    threadpool_limits = None

N_SPECIAL = 17  # 1 camera token + 16 register tokens per frame


@dataclass
class OracleParams:
    Wqkv: np.ndarray     # [3d, d] float64
    Wo: np.ndarray       # [d, d]  float64
    q_gamma: np.ndarray  # [H, Dh] float64
    q_beta: np.ndarray
    k_gamma: np.ndarray
    k_beta: np.ndarray
    H: int
    grid_h: int
    grid_w: int
    rope_base: float = 100.0
    ln_eps: float = 1e-5
    pos_offset: int = 0

    @property
    def d(self) -> int:
        return self.Wo.shape[0]

    @property
    def Dh(self) -> int:
        return self.d // self.H

    @property
    def T(self) -> int:
        return N_SPECIAL + self.grid_h * self.grid_w


def default_threads() -> int:
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, os.cpu_count() or 1)


# ----------------------------------------------------------------------------
# Token positions and RoPE
# ----------------------------------------------------------------------------

def token_positions(t_in_frame: np.ndarray, grid_w: int):
    """Map a token index inside its frame to (is_patch, grid row, grid column).

    Tokens 0..16 are the camera and register tokens (no position); token
    17 + p is patch p of the grid in row-major order.
    """
    t = np.asarray(t_in_frame, dtype=np.int64)
    is_patch = t >= N_SPECIAL
    p = np.where(is_patch, t - N_SPECIAL, 0)
    gw = max(grid_w, 1)  # a grid without patches has only special tokens
    return is_patch, p // gw, p % gw


def rope_angles(pos: np.ndarray, dh: int, base: float) -> np.ndarray:
    """Rotation angle pos * base**(-i/(Dh/4)) for each of the Dh/4 frequencies."""
    q4 = dh // 4
    theta = np.array([base ** (-(i / q4)) for i in range(q4)], dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope_2d(x: np.ndarray, t_in_frame: np.ndarray, grid_w: int, base: float,
            pos_offset: int = 0) -> np.ndarray:
    """Apply the 2D rotary encoding to x [M, H, Dh] (rows = tokens)."""
    M, H, Dh = x.shape
    q4 = Dh // 4
    is_patch, r, c = token_positions(t_in_frame, grid_w)
    out = x.copy()
    for half, pos in ((0, r + pos_offset), (1, c + pos_offset)):
        ang = rope_angles(pos, Dh, base)              # [M, q4]
        cos = np.cos(ang)[:, None, :]                 # broadcast over heads
        sin = np.sin(ang)[:, None, :]
        lo = half * 2 * q4
        a = x[:, :, lo:lo + q4]
        b = x[:, :, lo + q4:lo + 2 * q4]
        ra = a * cos - b * sin
        rb = b * cos + a * sin
        out[:, :, lo:lo + q4] = np.where(is_patch[:, None, None], ra, a)
        out[:, :, lo + q4:lo + 2 * q4] = np.where(is_patch[:, None, None], rb, b)
    return out


# ----------------------------------------------------------------------------
# QK LayerNorm, projection, attention
# ----------------------------------------------------------------------------

def layer_norm_heads(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                     eps: float) -> np.ndarray:
    """LayerNorm over the last axis of x [M, H, Dh], affine per head [H, Dh]."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)   # biased variance
    return (x - mu) / np.sqrt(var + eps) * gamma[None] + beta[None]


def _project(Xrows: np.ndarray, t_in_frame: np.ndarray, p: OracleParams,
             want=("q", "k", "v")):
    """Rows of X -> normalised, rotated q, k and raw v, each [M, H, Dh]."""
    d, H, Dh = p.d, p.H, p.Dh
    out = {}
    blocks = {"q": 0, "k": 1, "v": 2}
    for name in want:
        b = blocks[name]
        y = (Xrows @ p.Wqkv[b * d:(b + 1) * d].T).reshape(-1, H, Dh)
        if name == "q":
            y = layer_norm_heads(y, p.q_gamma, p.q_beta, p.ln_eps)
        elif name == "k":
            y = layer_norm_heads(y, p.k_gamma, p.k_beta, p.ln_eps)
        if name in ("q", "k"):
            y = rope_2d(y, t_in_frame, p.grid_w, p.rope_base, p.pos_offset)
        out[name] = y
    return out


def attention_probs(qh: np.ndarray, kh: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(Dh)) over the key axis, for one head."""
    a = (qh @ kh.T) / math.sqrt(qh.shape[-1])
    a = a - a.max(axis=1, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=1, keepdims=True)


def _attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, threads: int,
            chunk: int = 1024) -> np.ndarray:
    """Per-head softmax attention of the query rows q over keys k / values v.

    The work is split over (head, block of query rows) only; every row's
    softmax still spans all keys of the set.  Returns [Mq, H*Dh].
    """
    Mq, H, Dh = q.shape
    O = np.empty((Mq, H, Dh), dtype=np.float64)
    kh = [np.ascontiguousarray(k[:, h]) for h in range(H)]
    vh = [np.ascontiguousarray(v[:, h]) for h in range(H)]

    def job(h, lo):
        hi = min(Mq, lo + chunk)
        P = attention_probs(q[lo:hi, h], kh[h])
        O[lo:hi, h] = P @ vh[h]

    jobs = [(h, lo) for h in range(H) for lo in range(0, Mq, chunk)]
    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            job(*j)
    else:
        limiter = threadpool_limits(limits=1) if threadpool_limits else _NullCtx()
        with limiter, ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda j: job(*j), jobs))
    return O.reshape(Mq, H * Dh)


class _NullCtx:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def _check(X: np.ndarray, p: OracleParams):
    S, T, d = X.shape
    if T != p.T or d != p.d or d % p.H or p.Dh % 4:
        raise ValueError(f"shape mismatch: X {X.shape}, T={p.T}, d={p.d}, H={p.H}")
    return S, T, d


# ----------------------------------------------------------------------------
# The three block modes
# ----------------------------------------------------------------------------

def frame_attention(X: np.ndarray, p: OracleParams, threads: int | None = None) -> np.ndarray:
    """Frame block: attention among the T tokens of each frame separately."""
    threads = threads or default_threads()
    S, T, d = _check(X, p)
    Y = np.empty((S, T, d), dtype=np.float64)
    t = np.arange(T)
    for s in range(S):
        qkv = _project(X[s].astype(np.float64), t, p)
        O = _attend(qkv["q"], qkv["k"], qkv["v"], threads)
        Y[s] = O @ p.Wo.T
    return Y


def global_attention(X: np.ndarray, p: OracleParams, threads: int | None = None) -> np.ndarray:
    """Global mode: all S*T tokens form a single attention set."""
    threads = threads or default_threads()
    S, T, d = _check(X, p)
    Xf = X.reshape(S * T, d).astype(np.float64)
    t = np.tile(np.arange(T), S)
    qkv = _project(Xf, t, p)
    O = _attend(qkv["q"], qkv["k"], qkv["v"], threads)
    return (O @ p.Wo.T).reshape(S, T, d)


def register_attention(X: np.ndarray, p: OracleParams, threads: int | None = None) -> np.ndarray:
    """Register mode: the 17 special tokens of all frames form one set.

    Patch rows are passed through unchanged.
    """
    threads = threads or default_threads()
    S, T, d = _check(X, p)
    Y = X.astype(np.float64).copy()
    R = X[:, :N_SPECIAL].reshape(S * N_SPECIAL, d).astype(np.float64)
    t = np.tile(np.arange(N_SPECIAL), S)
    qkv = _project(R, t, p)
    O = _attend(qkv["q"], qkv["k"], qkv["v"], threads)
    Y[:, :N_SPECIAL] = (O @ p.Wo.T).reshape(S, N_SPECIAL, d)
    return Y


# ----------------------------------------------------------------------------
# Row-sampled variants (for sizes where the full oracle is too slow).  Each
# returns Y at the given flat row indices (row = s*T + t) and is the full
# definition restricted to those output rows: keys/values still span the set.
# ----------------------------------------------------------------------------

def global_attention_rows(X: np.ndarray, p: OracleParams, rows, threads: int | None = None) -> np.ndarray:
    threads = threads or default_threads()
    S, T, d = _check(X, p)
    rows = np.asarray(rows, dtype=np.int64)
    Xf = X.reshape(S * T, d)
    t_all = np.tile(np.arange(T), S)
    kv = _project(Xf.astype(np.float64), t_all, p, want=("k", "v"))
    q = _project(Xf[rows].astype(np.float64), t_all[rows], p, want=("q",))["q"]
    O = _attend(q, kv["k"], kv["v"], threads, chunk=64)
    return O @ p.Wo.T


def frame_attention_rows(X: np.ndarray, p: OracleParams, rows, threads: int | None = None) -> np.ndarray:
    threads = threads or default_threads()
    S, T, d = _check(X, p)
    rows = np.asarray(rows, dtype=np.int64)
    Y = np.empty((len(rows), d), dtype=np.float64)
    t = np.arange(T)
    for s in np.unique(rows // T):
        sel = np.nonzero(rows // T == s)[0]
        Xs = X[s].astype(np.float64)
        kv = _project(Xs, t, p, want=("k", "v"))
        tq = rows[sel] % T
        q = _project(Xs[tq], tq, p, want=("q",))["q"]
        Y[sel] = _attend(q, kv["k"], kv["v"], threads) @ p.Wo.T
    return Y


def register_attention_rows(X: np.ndarray, p: OracleParams, rows, threads: int | None = None) -> np.ndarray:
    threads = threads or default_threads()
    S, T, d = _check(X, p)
    rows = np.asarray(rows, dtype=np.int64)
    Xf = X.reshape(S * T, d)
    Y = Xf[rows].astype(np.float64).copy()
    spec = (rows % T) < N_SPECIAL
    if spec.any():
        R = X[:, :N_SPECIAL].reshape(S * N_SPECIAL, d).astype(np.float64)
        t = np.tile(np.arange(N_SPECIAL), S)
        kv = _project(R, t, p, want=("k", "v"))
        srows = (rows[spec] // T) * N_SPECIAL + rows[spec] % T
        q = _project(R[srows], t[srows], p, want=("q",))["q"]
        Y[spec] = _attend(q, kv["k"], kv["v"], threads) @ p.Wo.T
    return Y
