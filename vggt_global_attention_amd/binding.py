"""ctypes binding of libvggtattn: the C entry points under the same names.

Argument marshalling only -- every step of the computation runs in the HIP
library.  If the library is missing this module raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import contextlib

from .build import LIB, TUNE_LIB

OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE, EHIP, ERANGE, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
STATIC_SCRATCH_BYTES = 128 << 20
MODE_FRAME, MODE_GLOBAL, MODE_REGISTER, MODE_SUBSAMPLED, MODE_DESCRIPTOR, MODE_MERGED = \
    0, 1, 2, 3, 4, 5
STAGE_PREP, STAGE_QKV, STAGE_CORE, STAGE_OUT = 0, 1, 2, 3
STAGE_ALL = -1
STATUS_OFFSET = 16
RANGE_X, RANGE_WQKV, RANGE_WO, RANGE_AFFINE, RANGE_SCALE = 1, 2, 4, 8, 16
MODES = {"frame": MODE_FRAME, "global": MODE_GLOBAL, "register": MODE_REGISTER,
         "subsampled": MODE_SUBSAMPLED, "descriptor": MODE_DESCRIPTOR, "merged": MODE_MERGED}

EXPORTS = ("vggt_attn_workspace_bytes", "vggt_attn_frame", "vggt_attn_global",
           "vggt_attn_global_register", "vggt_attn_global_subsampled", "vggt_attn_global_rows",
           "vggt_attn_stage", "vggt_attn_bf16ops", "vggt_attn_subsampled_stage",
           "vggt_attn_global_rows_stage",
           "vggt_attn_global_merged", "vggt_attn_merged_stage",
           "vggt_attn_desc_cache_bytes", "vggt_attn_desc_cache_init", "vggt_attn_desc_append",
           "vggt_attn_desc_attend", "vggt_attn_desc_attend_stage",
           "vggt_attn_residual", "vggt_attn_schedule_workspace_bytes", "vggt_attn_schedule_run",
           "vggt_attn_range_status", "vggt_attn_block_noalloc", "vggt_attn_status_str",
           "vggt_attn_version")


class vggt_attn_shape(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("T", ctypes.c_int32), ("d", ctypes.c_int32),
                ("H", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("ln_eps", ctypes.c_float),
                ("pos_offset", ctypes.c_int32)]


class vggt_attn_block_weights(ctypes.Structure):
    _fields_ = [("Wqkv", ctypes.c_void_p), ("Wo", ctypes.c_void_p), ("q_gamma", ctypes.c_void_p),
                ("q_beta", ctypes.c_void_p), ("k_gamma", ctypes.c_void_p),
                ("k_beta", ctypes.c_void_p), ("layer_scale", ctypes.c_void_p)]


class vggt_attn_schedule(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("early_frame", ctypes.c_int32),
                ("register_layers", ctypes.c_uint64), ("cached_layers", ctypes.c_uint64),
                ("sub_h", ctypes.c_int32), ("sub_w", ctypes.c_int32),
                ("merge_frames", ctypes.c_int32), ("merge_win_h", ctypes.c_int32),
                ("merge_win_w", ctypes.c_int32), ("merge_r", ctypes.c_int32)]


class VggtAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


_lib = None
_tune_lib = None
_active = None  # the tuning build while inside tuning_build(), else None
_CALL_ARGS = [ctypes.POINTER(vggt_attn_shape)] + [ctypes.c_void_p] * 3 + [ctypes.c_void_p] * 4 + \
    [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]


def lib(path: str | None = None) -> ctypes.CDLL:
    """Load (once) the built library; raise if it is not there.  Inside
    tuning_build() this is the tuning build instead."""
    global _lib
    if _active is not None:
        return _active
    if _lib is not None:
        return _lib
    _lib = _load(path or LIB)
    return _lib


@contextlib.contextmanager
def tuning_build():
    """Route every call in the block through libvggtattn_tune.so, the build
    that honours the tuning environment variables (VGGT_ATTN_SPLIT,
    VGGT_ATTN_QB, VGGT_ATTN_WAVES, VGGT_GEMM, VGGT_GEMM_FGROUPS).  The
    product library ignores them."""
    global _tune_lib, _active
    if _tune_lib is None:
        _tune_lib = _load(TUNE_LIB)
    prev, _active = _active, _tune_lib
    try:
        yield _tune_lib
    finally:
        _active = prev


def _load(path: str) -> ctypes.CDLL:
    # torch wheels bundle their own HIP runtime: load it first so that the
    # library binds to the same runtime as torch's streams and allocations
    # (loaded the other way round, two runtimes coexist and launches fail).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"libvggtattn not built ({path} missing): run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    L.vggt_attn_workspace_bytes.restype = ctypes.c_size_t
    L.vggt_attn_workspace_bytes.argtypes = [ctypes.c_int, ctypes.POINTER(vggt_attn_shape)]
    for name in ("vggt_attn_frame", "vggt_attn_global", "vggt_attn_global_register"):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = _CALL_ARGS
    L.vggt_attn_stage.restype = ctypes.c_int
    L.vggt_attn_stage.argtypes = [ctypes.c_int, ctypes.c_int] + _CALL_ARGS
    L.vggt_attn_bf16ops.restype = ctypes.c_int
    L.vggt_attn_bf16ops.argtypes = [ctypes.c_int, ctypes.c_int] + _CALL_ARGS
    sub = [ctypes.POINTER(vggt_attn_shape), ctypes.c_int32, ctypes.c_int32] + _CALL_ARGS[1:]
    L.vggt_attn_global_subsampled.restype = ctypes.c_int
    L.vggt_attn_global_subsampled.argtypes = sub
    L.vggt_attn_subsampled_stage.restype = ctypes.c_int
    L.vggt_attn_subsampled_stage.argtypes = [ctypes.c_int] + sub
    mrg = [ctypes.POINTER(vggt_attn_shape)] + [ctypes.c_int32] * 4 + _CALL_ARGS[1:]
    L.vggt_attn_global_merged.restype = ctypes.c_int
    L.vggt_attn_global_merged.argtypes = mrg
    L.vggt_attn_merged_stage.restype = ctypes.c_int
    L.vggt_attn_merged_stage.argtypes = [ctypes.c_int] + mrg
    win = [ctypes.POINTER(vggt_attn_shape), ctypes.c_int64, ctypes.c_int64] + _CALL_ARGS[1:]
    L.vggt_attn_global_rows.restype = ctypes.c_int
    L.vggt_attn_global_rows.argtypes = win
    L.vggt_attn_global_rows_stage.restype = ctypes.c_int
    L.vggt_attn_global_rows_stage.argtypes = [ctypes.c_int] + win
    P, VP, I64, SZ = ctypes.POINTER(vggt_attn_shape), ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.vggt_attn_desc_cache_bytes.restype = ctypes.c_size_t
    L.vggt_attn_desc_cache_bytes.argtypes = [P, I64]
    L.vggt_attn_desc_cache_init.restype = ctypes.c_int
    L.vggt_attn_desc_cache_init.argtypes = [P, I64, VP, SZ, VP]
    L.vggt_attn_desc_append.restype = ctypes.c_int
    L.vggt_attn_desc_append.argtypes = [P, I64, I64, VP, I64, VP, VP, VP, VP, SZ, VP]
    attend = [P, I64, I64, VP, SZ, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
    L.vggt_attn_desc_attend.restype = ctypes.c_int
    L.vggt_attn_desc_attend.argtypes = attend
    L.vggt_attn_desc_attend_stage.restype = ctypes.c_int
    L.vggt_attn_desc_attend_stage.argtypes = [ctypes.c_int] + attend
    L.vggt_attn_residual.restype = ctypes.c_int
    L.vggt_attn_residual.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p]
    L.vggt_attn_schedule_workspace_bytes.restype = ctypes.c_size_t
    L.vggt_attn_schedule_workspace_bytes.argtypes = [ctypes.POINTER(vggt_attn_shape),
                                                     ctypes.POINTER(vggt_attn_schedule)]
    L.vggt_attn_schedule_run.restype = ctypes.c_int
    L.vggt_attn_schedule_run.argtypes = [ctypes.POINTER(vggt_attn_shape),
                                         ctypes.POINTER(vggt_attn_schedule),
                                         ctypes.POINTER(vggt_attn_block_weights), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
    L.vggt_attn_block_noalloc.restype = ctypes.c_int
    L.vggt_attn_block_noalloc.argtypes = [ctypes.c_int] + _CALL_ARGS[:9] + [ctypes.c_void_p]
    L.vggt_attn_range_status.restype = ctypes.c_int
    L.vggt_attn_range_status.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32),
                                         ctypes.c_void_p]
    L.vggt_attn_status_str.restype = ctypes.c_char_p
    L.vggt_attn_status_str.argtypes = [ctypes.c_int]
    L.vggt_attn_version.restype = ctypes.c_int
    L.vggt_attn_version.argtypes = []
    return L


def make_shape(S, T, d, H, grid_h, grid_w, rope_base=100.0, ln_eps=1e-5, pos_offset=0):
    return vggt_attn_shape(S, T, d, H, grid_h, grid_w, rope_base, ln_eps, pos_offset)


def vggt_attn_workspace_bytes(mode: int, shape: vggt_attn_shape) -> int:
    return lib().vggt_attn_workspace_bytes(mode, ctypes.byref(shape))


def _call(name, *args):
    return getattr(lib(), name)(*args)


def vggt_attn_frame(shape, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y, workspace,
                    workspace_bytes, stream) -> int:
    return _call("vggt_attn_frame", ctypes.byref(shape), X, Wqkv, Wo, q_gamma, q_beta,
                 k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_global(shape, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y, workspace,
                     workspace_bytes, stream) -> int:
    return _call("vggt_attn_global", ctypes.byref(shape), X, Wqkv, Wo, q_gamma, q_beta,
                 k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_global_register(shape, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y,
                              workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_global_register", ctypes.byref(shape), X, Wqkv, Wo, q_gamma,
                 q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_stage(mode, stage, shape, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y,
                    workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_stage", mode, stage, ctypes.byref(shape), X, Wqkv, Wo, q_gamma,
                 q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_bf16ops(mode, stage, shape, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y,
                      workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_bf16ops", mode, stage, ctypes.byref(shape), X, Wqkv, Wo, q_gamma,
                 q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_global_subsampled(shape, sub_h, sub_w, X, Wqkv, Wo, q_gamma, q_beta, k_gamma,
                                k_beta, Y, workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_global_subsampled", ctypes.byref(shape), sub_h, sub_w, X, Wqkv, Wo,
                 q_gamma, q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_subsampled_stage(stage, shape, sub_h, sub_w, X, Wqkv, Wo, q_gamma, q_beta,
                               k_gamma, k_beta, Y, workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_subsampled_stage", stage, ctypes.byref(shape), sub_h, sub_w, X, Wqkv,
                 Wo, q_gamma, q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_global_merged(shape, frames, win_h, win_w, r, X, Wqkv, Wo, q_gamma, q_beta,
                            k_gamma, k_beta, Y, workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_global_merged", ctypes.byref(shape), frames, win_h, win_w, r, X, Wqkv,
                 Wo, q_gamma, q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_merged_stage(stage, shape, frames, win_h, win_w, r, X, Wqkv, Wo, q_gamma, q_beta,
                           k_gamma, k_beta, Y, workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_merged_stage", stage, ctypes.byref(shape), frames, win_h, win_w, r, X,
                 Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_global_rows(shape, row_begin, row_count, X, Wqkv, Wo, q_gamma, q_beta, k_gamma,
                          k_beta, Y_rows, workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_global_rows", ctypes.byref(shape), row_begin, row_count, X, Wqkv, Wo,
                 q_gamma, q_beta, k_gamma, k_beta, Y_rows, workspace, workspace_bytes, stream)


def vggt_attn_global_rows_stage(stage, shape, row_begin, row_count, X, Wqkv, Wo, q_gamma,
                                q_beta, k_gamma, k_beta, Y_rows, workspace, workspace_bytes,
                                stream) -> int:
    return _call("vggt_attn_global_rows_stage", stage, ctypes.byref(shape), row_begin, row_count,
                 X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y_rows, workspace,
                 workspace_bytes, stream)


def vggt_attn_desc_cache_bytes(shape, capacity) -> int:
    return lib().vggt_attn_desc_cache_bytes(ctypes.byref(shape), capacity)


def vggt_attn_desc_cache_init(shape, capacity, cache, cache_bytes, stream) -> int:
    return _call("vggt_attn_desc_cache_init", ctypes.byref(shape), capacity, cache, cache_bytes,
                 stream)


def vggt_attn_desc_append(shape, capacity, count, D, m, Wqkv, k_gamma, k_beta, cache,
                          cache_bytes, stream) -> int:
    return _call("vggt_attn_desc_append", ctypes.byref(shape), capacity, count, D, m, Wqkv,
                 k_gamma, k_beta, cache, cache_bytes, stream)


def vggt_attn_desc_attend(shape, capacity, count, cache, cache_bytes, X, Wqkv, Wo, q_gamma,
                          q_beta, Y, workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_desc_attend", ctypes.byref(shape), capacity, count, cache,
                 cache_bytes, X, Wqkv, Wo, q_gamma, q_beta, Y, workspace, workspace_bytes, stream)


def vggt_attn_desc_attend_stage(stage, shape, capacity, count, cache, cache_bytes, X, Wqkv, Wo,
                                q_gamma, q_beta, Y, workspace, workspace_bytes, stream) -> int:
    return _call("vggt_attn_desc_attend_stage", stage, ctypes.byref(shape), capacity, count,
                 cache, cache_bytes, X, Wqkv, Wo, q_gamma, q_beta, Y, workspace,
                 workspace_bytes, stream)


def vggt_attn_residual(X, Y, Z, rows, d, gamma, period, active, C, c_stride, stream) -> int:
    return _call("vggt_attn_residual", X, Y, Z, rows, d, gamma, period, active, C, c_stride, stream)


def vggt_attn_schedule_workspace_bytes(shape, sched) -> int:
    return lib().vggt_attn_schedule_workspace_bytes(ctypes.byref(shape), ctypes.byref(sched))


def vggt_attn_schedule_run(shape, sched, blocks, X, state, caches, workspace, workspace_bytes,
                           stream) -> int:
    """`blocks` is a ctypes array of vggt_attn_block_weights (2 * n_layers)."""
    return _call("vggt_attn_schedule_run", ctypes.byref(shape), ctypes.byref(sched), blocks, X,
                 state, caches, workspace, workspace_bytes, stream)


def vggt_attn_block_noalloc(mode, shape, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y,
                            stream) -> int:
    return _call("vggt_attn_block_noalloc", mode, ctypes.byref(shape), X, Wqkv, Wo, q_gamma,
                 q_beta, k_gamma, k_beta, Y, stream)


def vggt_attn_range_status(workspace, stream) -> tuple:
    """(status, range bits) of the last call that used `workspace`."""
    bits = ctypes.c_uint32(0)
    st = _call("vggt_attn_range_status", workspace, ctypes.byref(bits), stream)
    return st, bits.value


def status_str(status: int) -> str:
    try:
        return lib().vggt_attn_status_str(status).decode()
    except Exception:
        return "?"


def vggt_attn_version() -> int:
    return lib().vggt_attn_version()
