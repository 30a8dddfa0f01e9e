"""Workload registry: the shapes the library is tested and measured on.

Each workload is one attention block of the VGGT Aggregator at a given frame
count.  Frames are 416x624 images cut into 16-pixel patches (26 x 39 = 1014
patches) plus 1 camera and 16 register tokens, so T = 1031 tokens per frame
("VGGT-Omega Aggregator explainer", ksqn.cn, sections 二 and 五).
"""

from __future__ import annotations

from dataclasses import dataclass

N_SPECIAL = 17


@dataclass(frozen=True)
class Workload:
    name: str
    cid: int            # seed namespace: seed = 1000 * cid + tensor index
    S: int              # frames
    grid_h: int
    grid_w: int
    d: int
    H: int
    modes: tuple        # block modes this workload is run in, in order
    dup_frames: int = 0  # frames replaced by a noisy copy of their predecessor
    rope_base: float = 100.0
    ln_eps: float = 1e-5

    @property
    def T(self) -> int:
        return N_SPECIAL + self.grid_h * self.grid_w

    @property
    def N(self) -> int:
        return self.S * self.T

    @property
    def R(self) -> int:
        return self.S * N_SPECIAL

    @property
    def Dh(self) -> int:
        return self.d // self.H

    def kept_keys(self, sub_h: int, sub_w: int) -> int:
        """Keys of subsampled global attention: 17 specials plus one patch per
        sub_h x sub_w window, in every frame."""
        return self.S * (N_SPECIAL + (-(-self.grid_h // sub_h)) * (-(-self.grid_w // sub_w)))

    def merged_tokens(self, frames: int, win_h: int, win_w: int, r: int) -> int:
        """Length of the merged sequence of HTTM merging: blocks of `frames`
        consecutive frames x win_h x win_w patch cells (cut at the ends), the
        first frame's patches of a block its destinations, the rest its
        sources, min(r, sources) merges per block; special tokens stay."""
        m = self.N
        for f0 in range(0, self.S, frames):
            nf = min(frames, self.S - f0)
            for r0 in range(0, self.grid_h, win_h):
                for c0 in range(0, self.grid_w, win_w):
                    cells = min(win_h, self.grid_h - r0) * min(win_w, self.grid_w - c0)
                    m -= min(r, (nf - 1) * cells)
        return m

    def attention_flop(self, mode: str, sub=(1, 1)) -> float:
        """4 * sum(L^2) * d over the attention sets of one block (2 FLOP per MAC);
        subsampled mode: 4 * N * (kept keys) * d (the two per-row extra columns
        are not counted); merged mode (sub = the four merge parameters): 4 M^2 d
        over the M merged tokens."""
        if mode == "subsampled":
            return 4.0 * self.N * self.kept_keys(*sub) * self.d
        if mode == "merged":
            return 4.0 * self.merged_tokens(*sub) ** 2 * self.d
        if mode == "frame":
            return 4.0 * self.S * self.T ** 2 * self.d
        if mode == "global":
            return 4.0 * self.N ** 2 * self.d
        if mode == "register":
            return 4.0 * self.R ** 2 * self.d
        raise ValueError(mode)

    def gemm_flop(self, mode: str) -> float:
        """QKV projection (6 M d^2) plus output projection (2 M d^2)."""
        M = self.R if mode == "register" else self.N
        return 8.0 * M * self.d ** 2

    def flop(self, mode: str, sub=(1, 1)) -> float:
        return self.attention_flop(mode, sub) + self.gemm_flop(mode)


WORKLOADS = {
    # tiny alternating block: the full oracle finishes in well under a second
    "tiny": Workload("tiny", 1, 2, 8, 8, 256, 4, ("frame", "global")),
    # VGGT scale, 24 frames (N = 24,744): global layer, also run as frame layer
    "s24": Workload("s24", 2, 24, 26, 39, 1024, 16, ("global", "frame")),
    # long global attention, 100 frames (N = 103,100): the measured workload
    "s100": Workload("s100", 3, 100, 26, 39, 1024, 16, ("global",)),
    # register mode at scale: frame over 500 x 1031, then 8,500 special tokens
    "s500": Workload("s500", 4, 500, 26, 39, 1024, 16, ("frame", "register")),
    # stress global attention, 300 frames (N = 309,300), 10% duplicated frames
    "s300": Workload("s300", 5, 300, 26, 39, 1024, 16, ("global",), dup_frames=30),
}


def custom(name: str, S: int, grid_h: int, grid_w: int, d: int, H: int,
           cid: int = 99, modes=("frame", "global", "register")) -> Workload:
    return Workload(name, cid, S, grid_h, grid_w, d, H, tuple(modes))
