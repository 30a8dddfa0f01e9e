"""fp64 CPU oracle of HTTM head-wise temporal token merging in the global block.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's CPU
baseline leg, never by the GPU library, and it shares no code with the HIP
path.  Float64 NumPy throughout; the q, k, v projections (QKV, per-head
LayerNorm, 2D RoPE) are those of `vggt_oracle`.

Source: "HTTM: Head-wise Temporal Token Merging for Faster VGGT" (article on
10100.com).  Section 02 lists the method's parts: head-wise merging (each
attention head merges tokens on its own), block-wise matching (tokens are
matched inside blocks instead of globally), temporal reordering (tokens are
regrouped into spatio-temporal blocks so that a block holds the same region of
consecutive frames) and head-wise adaptive outlier filtering.  Section 04
motivates the temporal blocks: the same spatial region of neighbouring frames
is highly similar.  Section 05: the merged Q, K and V sequences are shorter.

The page gives these ideas, not a rule.  The reading taken here, in the
page's order:

1. Temporal reordering.  Frames are grouped in consecutive runs of F
   ([0, F), [F, 2F), ...; the last run may be shorter) and the patch grid in
   windows of wh x ww cells (row-major; windows cut by the grid edge are
   smaller).  A block is one frame run x one window: its patch tokens, frame
   by frame, row-major inside the window.  Camera and register tokens are
   never merged.
2. Block-wise matching, per head.  In a block the destinations are the
   patches of the run's first frame and the sources those of its other
   frames.  The similarity of two tokens in a head is the dot product of
   their normalised, rotated keys there (the quantity attention compares keys
   by).  A source's best destination is the one of highest similarity (ties:
   the first); the r sources of highest best-similarity (ties: the first)
   merge into their best destinations, the others stay (a block with at most
   r sources merges them all).  These are decisions taken from floating
   point, so the oracle takes them in the kernels' precision: keys rounded to
   fp16 (to nearest, ties to even), their products summed in fp32 in feature
   order (`similarities`, an exact emulation: every product of two fp16
   values is exact in fp32, and an fp32 sum rounded from fp64 is the
   correctly rounded fp32 sum).  Everything else is fp64.
3. Head-wise merging.  Each head decides on its own keys.  A merged token is
   a destination together with the sources merged into it; its query, key and
   value are the means over its members and its size n is their count.
   Unmerged tokens have size 1.  The merged sequence is the same length in
   every head: N minus the merges of all blocks, min(r, sources) each.
4. Attention over the merged sequence, size-weighted: a merged key stands
   for its n members, so its softmax weight is n exp(logit), i.e.
   O_i = sum_j n_j exp(q_i . k_j / sqrt(Dh)) v_j / sum_j n_j exp(...).
5. Unmerging: every token takes, in each head, the output of its merged
   token; heads are concatenated and multiplied by Wo^T as in the global
   block.
The outlier filtering is left out: the page gives no rule for its budget.

With r = 0 nothing merges and the result is exactly the global block.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .vggt_oracle import N_SPECIAL, OracleParams, _check, _project, default_threads


@dataclass(frozen=True)
class HttmParams:
    frames: int   # F: frames per block
    win_h: int    # window rows
    win_w: int    # window columns
    r: int        # merges per block

    def check(self):
        if self.frames < 1 or self.win_h < 1 or self.win_w < 1 or self.r < 0:
            raise ValueError(f"bad HTTM parameters {self}")


def blocks(S: int, grid_h: int, grid_w: int, hp: HttmParams):
    """The spatio-temporal blocks (point 1), in order: frame run, then window
    row, then window column.  Each is (destinations, sources) as arrays of
    flat token indices s*T + t."""
    hp.check()
    T = N_SPECIAL + grid_h * grid_w
    out = []
    for f0 in range(0, S, hp.frames):
        run = range(f0, min(S, f0 + hp.frames))
        for r0 in range(0, grid_h, hp.win_h):
            for c0 in range(0, grid_w, hp.win_w):
                cells = [N_SPECIAL + r * grid_w + c
                         for r in range(r0, min(grid_h, r0 + hp.win_h))
                         for c in range(c0, min(grid_w, c0 + hp.win_w))]
                toks = [[s * T + t for t in cells] for s in run]
                dst = np.array(toks[0], dtype=np.int64)
                src = np.array([t for f in toks[1:] for t in f], dtype=np.int64)
                out.append((dst, src))
    return out


def merged_length(S: int, grid_h: int, grid_w: int, hp: HttmParams) -> int:
    N = S * (N_SPECIAL + grid_h * grid_w)
    return N - sum(min(hp.r, len(src)) for _, src in blocks(S, grid_h, grid_w, hp))


def fp16(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def similarities(ka: np.ndarray, kb: np.ndarray) -> np.ndarray:
    """fp32 dot products, summed in feature order, of fp16 keys: ka [..., s, F]
    against kb [..., d, F] -> [..., s, d] (values of fp32)."""
    a, b = fp16(ka), fp16(kb)
    acc = np.zeros(a.shape[:-1] + (b.shape[-2],), dtype=np.float32)
    for f in range(a.shape[-1]):
        prod = a[..., :, None, f] * b[..., None, :, f]   # exact: 11-bit x 11-bit significands
        acc = (acc.astype(np.float64) + prod).astype(np.float32)
    return acc.astype(np.float64)


def block_decisions(kh: np.ndarray, dst: np.ndarray, src: np.ndarray, r: int):
    """Point 2 for the blocks of one shape and one head: dst [B, nd] and src
    [B, ns] token indices; returns (best destination position per source,
    merged flag per source), both [B, ns], from the keys kh [N, Dh]."""
    B, ns = src.shape
    if ns == 0:
        return np.zeros((B, 0), dtype=np.int64), np.zeros((B, 0), dtype=bool)
    sim = similarities(kh[src], kh[dst])                 # [B, sources, destinations]
    best = np.argmax(sim, axis=2)                        # first of equal maxima
    score = np.take_along_axis(sim, best[..., None], axis=2)[..., 0]
    order = np.argsort(-score, axis=1, kind="stable")    # ties: the earlier source
    merged = np.zeros((B, ns), dtype=bool)
    np.put_along_axis(merged, order[:, :min(r, ns)], True, axis=1)
    return best, merged


def _block_shapes(S: int, grid_h: int, grid_w: int, hp: HttmParams):
    """The blocks grouped by shape: for each (nd, ns), the block numbers and
    their destination / source arrays, and every block's first merged index
    (the merged sequence: the 17 S special tokens, then block by block its
    destinations and its unmerged sources)."""
    bl = blocks(S, grid_h, grid_w, hp)
    base = np.empty(len(bl), dtype=np.int64)
    pos = S * N_SPECIAL
    shapes = {}
    for b, (dst, src) in enumerate(bl):
        base[b] = pos
        pos += len(dst) + len(src) - min(hp.r, len(src))
        shapes.setdefault((len(dst), len(src)), []).append(b)
    out = []
    for (nd, ns), ids in shapes.items():
        out.append((np.array(ids), np.stack([bl[b][0] for b in ids]).reshape(len(ids), nd),
                    np.stack([bl[b][1] for b in ids]).reshape(len(ids), ns)))
    return out, base, pos


def head_owner(kh: np.ndarray, S: int, grid_h: int, grid_w: int, hp: HttmParams):
    """One head's merging (points 1-3): the merged token owning each token,
    owner [N], and the merged tokens' sizes n [M].  Merged order: the special
    tokens frame by frame, then block by block each destination (with the
    sources merged into it) and the block's unmerged sources in order."""
    T = N_SPECIAL + grid_h * grid_w
    N = S * T
    owner = np.full(N, -1, dtype=np.int64)
    t = np.arange(N)
    spec = (t % T) < N_SPECIAL
    owner[spec] = (t[spec] // T) * N_SPECIAL + t[spec] % T
    shapes, base, M = _block_shapes(S, grid_h, grid_w, hp)
    for ids, dst, src in shapes:
        nd = dst.shape[1]
        b0 = base[ids][:, None]
        owner[dst] = b0 + np.arange(nd)[None, :]
        best, merged = block_decisions(kh, dst, src, hp.r)
        stay = np.cumsum(~merged, axis=1) - 1            # rank among the unmerged sources
        owner[src] = np.where(merged, b0 + best, b0 + nd + stay)
    assert (owner >= 0).all()
    n = np.bincount(owner, minlength=M).astype(np.float64)
    return owner, n


def head_groups(kh: np.ndarray, S: int, grid_h: int, grid_w: int, hp: HttmParams):
    """head_owner as member lists, in merged order."""
    owner, n = head_owner(kh, S, grid_h, grid_w, hp)
    order = np.argsort(owner, kind="stable")
    return np.split(order, np.cumsum(n.astype(np.int64))[:-1])


def merged_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, owner: np.ndarray,
                     n: np.ndarray, query_groups=None) -> np.ndarray:
    """Points 3 and 4 for one head: means over the members, then the
    size-weighted softmax.  q, k, v [N, Dh]; returns the output of every
    merged token (or of those listed in query_groups) [G, Dh]."""
    def mean(x):
        acc = np.zeros((len(n), x.shape[1]))
        np.add.at(acc, owner, x)
        return acc / n[:, None]
    qm, km, vm = mean(q), mean(k), mean(v)
    if query_groups is not None:
        qm = qm[query_groups]
    out = np.empty((len(qm), q.shape[1]))
    for lo in range(0, len(qm), 2048):
        a = (qm[lo:lo + 2048] @ km.T) / math.sqrt(q.shape[-1]) + np.log(n)[None, :]
        a -= a.max(axis=1, keepdims=True)
        w = np.exp(a)
        out[lo:lo + 2048] = (w @ vm) / w.sum(axis=1, keepdims=True)
    return out


def _qkv(X: np.ndarray, p: OracleParams, want=("q", "k", "v")):
    S, T, d = _check(X, p)
    Xf = X.reshape(S * T, d).astype(np.float64)
    return _project(Xf, np.tile(np.arange(T), S), p, want=want)


def httm_attention(X: np.ndarray, p: OracleParams, hp: HttmParams, threads=None) -> np.ndarray:
    """The global block with HTTM merging (points 1-5): Y [S, T, d]."""
    S, T, d = _check(X, p)
    f = _qkv(X, p)
    N = S * T
    O = np.empty((N, p.H, p.Dh))
    for h in range(p.H):
        owner, n = head_owner(f["k"][:, h], S, p.grid_h, p.grid_w, hp)
        og = merged_attention(f["q"][:, h], f["k"][:, h], f["v"][:, h], owner, n)
        O[:, h] = og[owner]                      # point 5: unmerge
    return (O.reshape(N, d) @ p.Wo.T).reshape(S, T, d)


def httm_attention_rows(X: np.ndarray, p: OracleParams, hp: HttmParams, rows,
                        threads=None) -> np.ndarray:
    """Y at the flat rows `rows`: merging and keys over the whole set, the
    queries of only the merged tokens those rows belong to."""
    S, T, d = _check(X, p)
    N = S * T
    rows = np.asarray(rows, dtype=np.int64)
    f = _qkv(X, p, want=("k", "v"))
    heads = []
    members = np.zeros(N, dtype=bool)          # tokens whose query some merged query needs
    for h in range(p.H):
        owner, n = head_owner(f["k"][:, h], S, p.grid_h, p.grid_w, hp)
        need, back = np.unique(owner[rows], return_inverse=True)
        members |= np.isin(owner, need)
        heads.append((owner, n, need, back))
    q = np.zeros((N, p.H, p.Dh))
    idx = np.flatnonzero(members)
    q[idx] = _project(X.reshape(N, d).astype(np.float64)[idx], idx % T, p, want=("q",))["q"]
    O = np.empty((len(rows), p.H, p.Dh))
    for h, (owner, n, need, back) in enumerate(heads):
        og = merged_attention(q[:, h], f["k"][:, h], f["v"][:, h], owner, n, need)
        O[:, h] = og[back]
    return O.reshape(len(rows), d) @ p.Wo.T


def fragile(X: np.ndarray, p: OracleParams, hp: HttmParams, rel: float = 2.0 ** -8,
            terms: int = 2, rows=None):
    """(token, head) pairs whose merged token a GPU computation could make
    differ from the oracle's.  The kernels decide from the same fp16 keys and
    fp32 sums as `similarities` wherever their fp16 keys equal the oracle's
    rounding of its fp64 keys; a key element can come out one fp16 unit (at
    most 2^-10 of it) apart where their fp32 arithmetic lands on the other
    side of a rounding boundary.  A decision is fragile when it is closer than
    rel times the sum of the `terms` largest |k_a,i k_b,i| of each of the two
    similarities involved (room for a few such elements): a source's best
    destination against its runner-up, or the split between the r merged
    sources of a block and the rest.  All tokens of such a block are flagged
    in that head.  Boolean [S*T, H], or [len(rows), H] for the flat token
    indices `rows` (then only the blocks holding them are looked at)."""
    S, T, d = _check(X, p)
    N = S * T
    shapes, _, _ = _block_shapes(S, p.grid_h, p.grid_w, hp)
    if rows is None:
        k = _qkv(X, p, want=("k",))["k"]
    else:
        rows = np.asarray(rows, dtype=np.int64)
        hit = np.zeros(N, dtype=bool)
        hit[rows] = True
        keep = []
        for ids, dst, src in shapes:
            sel = hit[dst].any(axis=1) | hit[src].any(axis=1)
            keep.append((ids[sel], dst[sel], src[sel]))
        shapes = keep
        need = np.unique(np.concatenate([np.concatenate([dst.ravel(), src.ravel()])
                                         for _, dst, src in shapes] + [np.zeros(0, np.int64)]))
        k = np.zeros((N, p.H, p.Dh))
        if len(need):
            Xf = X.reshape(N, d).astype(np.float64)
            k[need] = _project(Xf[need], need % T, p, want=("k",))["k"]
    frag = np.zeros((N, p.H), dtype=bool)
    for h in range(p.H):
        kh16 = fp16(k[:, h])
        for ids, dst, src in shapes:
            B, ns = src.shape
            nd = dst.shape[1]
            if ns == 0:
                continue
            sim = similarities(kh16[src], kh16[dst])                  # [B, ns, nd]
            prod = np.abs(kh16[src][:, :, None, :] * kh16[dst][:, None, :, :])
            eps = rel * np.sort(prod, axis=-1)[..., -terms:].sum(axis=-1)
            best = np.argmax(sim, axis=2)
            score = np.take_along_axis(sim, best[..., None], axis=2)[..., 0]
            e_best = np.take_along_axis(eps, best[..., None], axis=2)[..., 0]
            bad = np.zeros(B, dtype=bool)
            if nd > 1:
                gap = (score - e_best)[..., None] - (sim + eps)
                np.put_along_axis(gap, best[..., None], np.inf, axis=2)
                bad |= (gap <= 0).any(axis=(1, 2))
            r = min(hp.r, ns)
            if 0 < r < ns:
                order = np.argsort(-score, axis=1, kind="stable")
                lo = np.take_along_axis(score - e_best, order[:, :r], axis=1).min(axis=1)
                hi = np.take_along_axis(score + e_best, order[:, r:], axis=1).max(axis=1)
                bad |= lo <= hi
            frag[dst[bad].ravel(), h] = True
            frag[src[bad].ravel(), h] = True
    return frag if rows is None else frag[rows]
