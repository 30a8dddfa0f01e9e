"""C-ABI contract checks that need no GPU: exports, workspace sizing, and every
argument error path (all of which return before the first HIP call)."""

from __future__ import annotations

import os
import re

import pytest

from vggt_global_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libvggtattn.h")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(vggt_attn_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for need in ("vggt_attn_frame", "vggt_attn_global", "vggt_attn_global_register",
                 "vggt_attn_workspace_bytes", "vggt_attn_status_str"):
        assert need in fns


def test_library_exports_every_header_symbol():
    L = B.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) == set(B.EXPORTS)


def shape(**kw):
    base = dict(S=100, T=1031, d=1024, H=16, grid_h=26, grid_w=39)
    base.update(kw)
    return B.make_shape(**base)


def test_workspace_bytes():
    s = shape()
    g = B.vggt_attn_workspace_bytes(B.MODE_GLOBAL, s)
    f = B.vggt_attn_workspace_bytes(B.MODE_FRAME, s)
    r = B.vggt_attn_workspace_bytes(B.MODE_REGISTER, s)
    N = 100 * 1031
    assert g >= 3 * 16 * N * 64 * 2          # q, k, v in fp16 for every token and head
    assert f >= g                            # frames are padded to whole key tiles
    assert 0 < r < g / 40                    # only 17 of 1031 rows per frame
    assert B.vggt_attn_workspace_bytes(7, s) == 0
    assert B.vggt_attn_workspace_bytes(B.MODE_GLOBAL, shape(T=1030)) == 0


FAKE = dict(X=0x100000, Wqkv=0x200000, Wo=0x300000, qg=0x400000, qb=0x400100, kg=0x400200,
            kb=0x400300, Y=0x500000)


def call(fn, s, ws_bytes=None, ws=0x10000000, **over):
    a = dict(FAKE)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = B.vggt_attn_workspace_bytes(B.MODE_GLOBAL, s) or 1 << 30
    return fn(s, a["X"], a["Wqkv"], a["Wo"], a["qg"], a["qb"], a["kg"], a["kb"], a["Y"], ws,
              ws_bytes, None)


TINY = dict(S=2, T=81, d=256, H=4, grid_h=8, grid_w=8)


@pytest.mark.parametrize("bad,code", [
    (dict(T=80), B.ESHAPE),                 # T != 17 + grid_h*grid_w
    (dict(d=192, H=3), B.ESHAPE),           # d not a multiple of 128
    (dict(d=256, H=8), B.ESHAPE),           # Dh = 32
    (dict(S=0), B.ESHAPE),
    (dict(grid_h=-1, T=17 - 8), B.ESHAPE),
    (dict(rope_base=0.0), B.ERANGE),
    (dict(rope_base=float("inf")), B.ERANGE),
    (dict(ln_eps=-1.0), B.ERANGE),
    (dict(pos_offset=-3), B.ERANGE),
])
def test_shape_errors(bad, code):
    kw = dict(TINY)
    kw.update(bad)
    s = B.make_shape(**kw)
    for fn in (B.vggt_attn_frame, B.vggt_attn_global, B.vggt_attn_global_register):
        assert call(fn, s, ws_bytes=1 << 30) == code


def test_pointer_errors():
    s = B.make_shape(**TINY)
    for fn in (B.vggt_attn_frame, B.vggt_attn_global, B.vggt_attn_global_register):
        assert call(fn, s, X=0) == B.EINVAL
        assert call(fn, s, kb=0) == B.EINVAL
        assert call(fn, s, ws=0) == B.EINVAL
        assert call(fn, s, X=0x100008) == B.EALIGN
        assert call(fn, s, qg=0x400002) == B.EALIGN
        assert call(fn, s, ws=0x10000080) == B.EALIGN
        assert call(fn, s, ws_bytes=1024) == B.EWORKSPACE
        assert call(fn, s, Y=0x100000 + 64) == B.EINVAL       # Y overlaps X
        assert call(fn, s, Y=0x10000000) == B.EINVAL          # Y overlaps the workspace
        assert call(fn, s, ws=0x300000) == B.EINVAL           # workspace holds Wo


def test_stage_errors():
    s = B.make_shape(**TINY)
    a = [FAKE[k] for k in ("X", "Wqkv", "Wo", "qg", "qb", "kg", "kb", "Y")]
    assert B.vggt_attn_stage(B.MODE_GLOBAL, 9, s, *a, 0x10000000, 1 << 30, None) == B.EINVAL
    assert B.vggt_attn_stage(5, B.STAGE_CORE, s, *a, 0x10000000, 1 << 30, None) == B.EINVAL
    assert B.vggt_attn_stage(B.MODE_GLOBAL, B.STAGE_CORE, s, *a, 0x10000000, 16, None) == B.EWORKSPACE


def test_status_strings():
    for code in (B.OK, B.EINVAL, B.ESHAPE, B.EALIGN, B.EWORKSPACE, B.EHIP, B.ERANGE):
        assert B.status_str(code) and B.status_str(code) != "unknown status"
    assert B.status_str(12345) == "unknown status"
    assert B.vggt_attn_version() >= 10000


# ----------------------------------------------------------------------------
# Subsampled global attention entry points
# ----------------------------------------------------------------------------

def sub_fn(sub_h, sub_w):
    def fn(s, *rest):
        return B.vggt_attn_global_subsampled(s, sub_h, sub_w, *rest)
    return fn


def test_subsampled_workspace_bytes():
    s = shape()
    g = B.vggt_attn_workspace_bytes(B.MODE_GLOBAL, s)
    sub = B.vggt_attn_workspace_bytes(B.MODE_SUBSAMPLED, s)
    N = 100 * 1031
    # compact keys / values sized for every window choice (1 x 1 keeps all tokens)
    assert sub >= g + 2 * 16 * N * 64 * 2
    assert B.vggt_attn_workspace_bytes(B.MODE_SUBSAMPLED, shape(T=1030)) == 0


def test_subsampled_errors():
    s = B.make_shape(**TINY)
    big = B.vggt_attn_workspace_bytes(B.MODE_SUBSAMPLED, s)
    for sh, sw in ((0, 3), (3, 0), (-1, 1)):
        assert call(sub_fn(sh, sw), s, ws_bytes=big) == B.ERANGE
    fn = sub_fn(3, 3)
    assert call(fn, s, ws_bytes=big, X=0) == B.EINVAL
    assert call(fn, s, ws_bytes=big, X=0x100008) == B.EALIGN
    assert call(fn, s, ws_bytes=big - 256) == B.EWORKSPACE
    # the global mode's workspace is too small for the compact key / value copies
    assert call(fn, s) == B.EWORKSPACE
    assert call(fn, s, ws_bytes=big, Y=0x100000 + 64) == B.EINVAL
    bad = dict(TINY)
    bad.update(T=80)
    assert call(fn, B.make_shape(**bad), ws_bytes=big) == B.ESHAPE


def test_subsampled_stage_errors():
    s = B.make_shape(**TINY)
    a = [FAKE[k] for k in ("X", "Wqkv", "Wo", "qg", "qb", "kg", "kb", "Y")]
    big = B.vggt_attn_workspace_bytes(B.MODE_SUBSAMPLED, s)
    # the generic stage entry has no windows to pass
    assert B.vggt_attn_stage(B.MODE_SUBSAMPLED, B.STAGE_CORE, s, *a, 0x10000000, big,
                             None) == B.EINVAL
    assert B.vggt_attn_subsampled_stage(7, s, 3, 3, *a, 0x10000000, big, None) == B.EINVAL
    assert B.vggt_attn_subsampled_stage(B.STAGE_CORE, s, 0, 3, *a, 0x10000000, big,
                                        None) == B.ERANGE
    assert B.vggt_attn_subsampled_stage(B.STAGE_CORE, s, 3, 3, *a, 0x10000000, 16,
                                        None) == B.EWORKSPACE


# ----------------------------------------------------------------------------
# Query-row window of the global block
# ----------------------------------------------------------------------------

def rows_fn(begin, count):
    def fn(s, *rest):
        return B.vggt_attn_global_rows(s, begin, count, *rest)
    return fn


def test_global_rows_errors():
    s = B.make_shape(**TINY)               # N = 162
    ws = B.vggt_attn_workspace_bytes(B.MODE_GLOBAL, s)
    for begin, count in ((-1, 10), (0, 0), (0, -5), (100, 63), (162, 1), (0, 163)):
        assert call(rows_fn(begin, count), s, ws_bytes=ws) == B.ERANGE, (begin, count)
    fn = rows_fn(10, 20)
    assert call(fn, s, ws_bytes=ws, X=0) == B.EINVAL
    assert call(fn, s, ws_bytes=ws, Y=0x100008) == B.EALIGN
    assert call(fn, s, ws_bytes=ws - 256) == B.EWORKSPACE
    # Y holds 20 rows x 256 features x 2 bytes: overlapping X's first bytes is rejected,
    # ending right before X is fine (the call then fails only later, on the fake pointers,
    # so check the aliasing verdict through a too-small workspace instead)
    assert call(fn, s, ws_bytes=ws, Y=0x100000 - 20 * 256 * 2 + 16) == B.EINVAL
    assert call(fn, s, ws_bytes=16, Y=0x100000 - 20 * 256 * 2) == B.EWORKSPACE
    a = [FAKE[k] for k in ("X", "Wqkv", "Wo", "qg", "qb", "kg", "kb", "Y")]
    assert B.vggt_attn_global_rows_stage(9, s, 0, 10, *a, 0x10000000, ws, None) == B.EINVAL
    assert B.vggt_attn_global_rows_stage(B.STAGE_CORE, s, 0, 0, *a, 0x10000000, ws,
                                         None) == B.ERANGE
