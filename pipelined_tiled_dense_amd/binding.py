"""Thin ctypes binding over the C ABI of ``libgemm_bf16.so`` (include/gemm_bf16.h).

Every function here only marshals arguments: the GEMM itself runs in the HIP
kernels of the library.  There is no fallback: if the library is missing or
cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libgemm_bf16.so")

GEMM_OK = 0
GEMM_ERR_INVALID_VALUE = -1
GEMM_ERR_MISALIGNED = -2
GEMM_ERR_UNSUPPORTED_SHAPE = -3
GEMM_ERR_STAGES = -4
GEMM_ERR_SYNC_MODE = -5
GEMM_ERR_DEVICE = -6
GEMM_ERR_LAUNCH = -7
GEMM_ERR_ALIAS = -8
GEMM_ERR_SCRATCH = -9
GEMM_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

SYNC_MODES = {"barrier": 0, "flags": 1, "wavespec": 2, "pingpong": 3}
STAGES_WINDOWS = 5          # GEMM_STAGES_WINDOWS: the split-window ring (barrier sync)


class GemmError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__("%s%s (status %d)" % (what + ": " if what else "", strerror(code), code))


class Plan(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("sync_mode", ctypes.c_int32),
                ("b_transposed", ctypes.c_int32), ("mfma_waves", ctypes.c_int32),
                ("producer_waves", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("tiles", ctypes.c_int64),
                ("k_steps", ctypes.c_int64), ("grid", ctypes.c_int64),
                ("k_splits", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("tail_tiles", ctypes.c_int64), ("tail_splits", ctypes.c_int64),
                ("pad_bytes", ctypes.c_int64), ("mfma_block", ctypes.c_int64),
                ("pipelines", ctypes.c_int64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError("HIP library %s is not built; run __graft_entry__.build() or "
                               "python -m pipelined_tiled_dense_amd.build" % LIBRARY)
        lib = ctypes.CDLL(LIBRARY)
        i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        sig = [i64, i64, i64, p, i64, p, i64, p, i64, i32, i32, p]
        lib.gemm_bf16.argtypes = sig
        lib.gemm_bf16.restype = i32
        lib.gemm_bf16_bt.argtypes = sig
        lib.gemm_bf16_bt.restype = i32
        lib.gemm_bf16_noalloc.argtypes = sig
        lib.gemm_bf16_noalloc.restype = i32
        lib.gemm_bf16_plan.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(Plan)]
        lib.gemm_bf16_plan.restype = i32
        lib.gemm_bf16_plan_cus.argtypes = [i64, i64, i64, i32, i32, i32, i32, ctypes.POINTER(Plan)]
        lib.gemm_bf16_plan_cus.restype = i32
        lib.gemm_bf16_strerror.argtypes = [i32]
        lib.gemm_bf16_strerror.restype = ctypes.c_char_p
        lib.gemm_bf16_sync_timeouts.argtypes = [i32]
        lib.gemm_bf16_sync_timeouts.restype = i64
        lib.gemm_bf16_set_sync_spin_limit.argtypes = [i64]
        lib.gemm_bf16_set_sync_spin_limit.restype = i64
        lib.gemm_bf16_set_clock_sampling.argtypes = [i32]
        lib.gemm_bf16_set_clock_sampling.restype = i32
        lib.gemm_bf16_clock_samples.argtypes = [ctypes.POINTER(ctypes.c_uint64), i32]
        lib.gemm_bf16_clock_samples.restype = i32
        lib.gemm_bf16_workspace_info.argtypes = [ctypes.POINTER(ctypes.c_int64)] * 3
        lib.gemm_bf16_workspace_info.restype = i32
        lib.gemm_bf16_release_workspaces.argtypes = []
        lib.gemm_bf16_release_workspaces.restype = i32
        _lib = lib
    return _lib


# -- the C entry points, same names --------------------------------------------
def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream) -> int:
    return library().gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream)


def gemm_bf16_bt(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream) -> int:
    return library().gemm_bf16_bt(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream)


def gemm_bf16_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream) -> int:
    return library().gemm_bf16_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream)


def gemm_bf16_plan(M, N, K, b_transposed, stages, sync_mode) -> dict:
    out = Plan()
    rc = library().gemm_bf16_plan(M, N, K, int(bool(b_transposed)), stages, sync_mode,
                                  ctypes.byref(out))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_bf16_plan")
    return out.as_dict()


def gemm_bf16_plan_cus(M, N, K, b_transposed, stages, sync_mode, compute_units) -> dict:
    out = Plan()
    rc = library().gemm_bf16_plan_cus(M, N, K, int(bool(b_transposed)), stages, sync_mode, compute_units,
                                      ctypes.byref(out))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_bf16_plan_cus")
    return out.as_dict()


def gemm_bf16_strerror(code: int) -> str:
    return library().gemm_bf16_strerror(code).decode()


def gemm_bf16_sync_timeouts(reset: bool = False) -> int:
    n = library().gemm_bf16_sync_timeouts(int(bool(reset)))
    if n < 0:
        raise GemmError(int(n), "gemm_bf16_sync_timeouts")
    return int(n)


def gemm_bf16_set_sync_spin_limit(polls: int) -> int:
    n = library().gemm_bf16_set_sync_spin_limit(int(polls))
    if n < 0:
        raise GemmError(int(n), "gemm_bf16_set_sync_spin_limit")
    return int(n)


def gemm_bf16_workspace_info() -> dict:
    """The temporary memory the library keeps on the current device: blocks,
    their total bytes, and how many are taken right now."""
    blocks, nbytes, busy = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = library().gemm_bf16_workspace_info(ctypes.byref(blocks), ctypes.byref(nbytes), ctypes.byref(busy))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_bf16_workspace_info")
    return {"blocks": blocks.value, "bytes": nbytes.value, "busy": busy.value}


def gemm_bf16_release_workspaces() -> None:
    """Frees the temporary memory the library keeps on the current device
    (synchronises the device)."""
    rc = library().gemm_bf16_release_workspaces()
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_bf16_release_workspaces")


def gemm_bf16_set_clock_sampling(enable: bool) -> bool:
    """Turns the kernels' clock sampling on or off; returns the previous setting."""
    return bool(library().gemm_bf16_set_clock_sampling(int(bool(enable))))


def gemm_bf16_clock_samples(reset: bool = False) -> dict:
    """The current device's clock sums: shader-clock ticks, constant-rate ticks,
    samples, the constant rate in Hz, and the mean clock in GHz they give
    (None without samples)."""
    out = (ctypes.c_uint64 * 4)()
    rc = library().gemm_bf16_clock_samples(out, int(bool(reset)))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_bf16_clock_samples")
    shader, wall, n, hz = (int(v) for v in out)
    return {"shader_ticks": shader, "wall_ticks": wall, "samples": n, "wall_hz": hz,
            "clock_ghz": shader / wall * hz / 1e9 if wall > 0 else None}


strerror = gemm_bf16_strerror


# -- tensor-level convenience ----------------------------------------------------
def _sync_code(sync) -> int:
    if isinstance(sync, str):
        if sync not in SYNC_MODES:
            raise ValueError("sync must be one of %s" % sorted(SYNC_MODES))
        return SYNC_MODES[sync]
    return int(sync)


def gemm(A, B, *, b_transposed: bool = False, stages: int = 0, sync="barrier", out=None,
         stream=None):
    """C = A @ B (or A @ B.T-stored when ``b_transposed``) for CUDA bf16 tensors
    with unit inner stride.  Returns ``out`` (allocated if None).  Runs on the
    current stream unless a torch stream is given."""
    import torch

    for name, X in (("A", A), ("B", B)):
        if X.dtype != torch.bfloat16 or X.dim() != 2 or not X.is_cuda:
            raise TypeError("%s must be a 2-D bfloat16 CUDA tensor" % name)
        if X.shape[0] * X.shape[1] > 0 and X.stride(1) != 1:
            raise ValueError("%s needs unit stride along its second dimension" % name)
    M, K = A.shape
    if b_transposed:
        N, KB = B.shape
    else:
        KB, N = B.shape
    if KB != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, KB))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or (M * N > 0 and out.stride(1) != 1):
        raise ValueError("out must be a bfloat16 tensor of shape (M, N) with unit inner stride")
    s = (stream or torch.cuda.current_stream(A.device)).cuda_stream
    fn = gemm_bf16_bt if b_transposed else gemm_bf16
    lda = A.stride(0) if M > 1 else max(K, 8)
    ldb = B.stride(0) if B.shape[0] > 1 else max(B.shape[1], 8)
    ldc = out.stride(0) if M > 1 else max(N, 8)
    rc = fn(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc,
            int(stages), _sync_code(sync), s)
    if rc != GEMM_OK:
        raise GemmError(rc, fn.__name__)
    return out
