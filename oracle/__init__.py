"""CPU oracle for the bf16 GEMM (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and the two share no code.

The arithmetic lives in ``oracle_gemm.c`` (plain C, fp64 accumulation in
increasing k, one round-to-nearest-even to bf16).  This module only builds that
file with gcc and marshals numpy arrays of bf16 bit patterns (``uint16``) into
it.  The problem statement it follows is the matmul of "Allow separate sub-DAG
for load and compute warp groups with warp-specialized circular buffering",
section "Pseudo-code" (fp32 accumulate, results converted to bf16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle_gemm.c")
LIBRARY = os.path.join(_HERE, "liboracle_gemm.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = output + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source, "-lm"], check=True)
    os.replace(tmp, output)
    return output


class Oracle:
    """ctypes view of one built copy of ``oracle_gemm.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm_f64.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_int, p, i64]
        lib.oracle_gemm_f64.restype = ctypes.c_int
        lib.oracle_gemm_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_int, p, i64]
        lib.oracle_gemm_bf16.restype = ctypes.c_int
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_round_array.argtypes = [i64, p, p]
        lib.oracle_round_array.restype = None
        lib.oracle_decode_array.argtypes = [i64, p, p]
        lib.oracle_decode_array.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _check_operands(A, B, K, N, b_transposed):
        if A.dtype != np.uint16 or B.dtype != np.uint16:
            raise TypeError("operands must be uint16 arrays of bf16 bit patterns")
        if A.ndim != 2 or B.ndim != 2:
            raise ValueError("operands must be 2-D")
        if A.shape[1] < K:
            raise ValueError("A has fewer than K columns")
        if b_transposed:
            if B.shape[0] < N or B.shape[1] < K:
                raise ValueError("B (N x K) too small")
        elif B.shape[0] < K or B.shape[1] < N:
            raise ValueError("B (K x N) too small")
        for X in (A, B):
            if X.strides[1] != 2:
                raise ValueError("operands need unit inner stride")

    def _shape(self, A, B, b_transposed, K=None, N=None):
        M = A.shape[0]
        if K is None:
            K = B.shape[1] if b_transposed else B.shape[0]
        if N is None:
            N = B.shape[0] if b_transposed else B.shape[1]
        return M, N, K

    # -- API ---------------------------------------------------------------
    def gemm_bf16(self, A: np.ndarray, B: np.ndarray, b_transposed: bool = False,
                  K: int | None = None, N: int | None = None) -> np.ndarray:
        """C = round_bf16(A @ B) as uint16 bits.  A is M x (>=K) with row stride
        from its strides; B is K x N (or N x K when ``b_transposed``)."""
        M, N, K = self._shape(A, B, b_transposed, K, N)
        self._check_operands(A, B, K, N, b_transposed)
        C = np.zeros((M, N), dtype=np.uint16)
        rc = self.lib.oracle_gemm_bf16(M, N, K, A.ctypes.data, A.strides[0] // 2,
                                       B.ctypes.data, B.strides[0] // 2, int(bool(b_transposed)),
                                       C.ctypes.data, N)
        if rc != 0:
            raise MemoryError("oracle row buffer allocation failed")
        return C

    def gemm_f64(self, A: np.ndarray, B: np.ndarray, b_transposed: bool = False,
                 K: int | None = None, N: int | None = None) -> np.ndarray:
        """The same sums before rounding, as float64."""
        M, N, K = self._shape(A, B, b_transposed, K, N)
        self._check_operands(A, B, K, N, b_transposed)
        C = np.zeros((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_f64(M, N, K, A.ctypes.data, A.strides[0] // 2,
                                      B.ctypes.data, B.strides[0] // 2, int(bool(b_transposed)),
                                      C.ctypes.data, N)
        if rc != 0:
            raise MemoryError("oracle row buffer allocation failed")
        return C

    def f64_to_bf16(self, x) -> np.ndarray:
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_round_array(x.size, x.ctypes.data, out.ctypes.data)
        return out

    def decode(self, bits) -> np.ndarray:
        """Exact fp64 values of bf16 bit patterns, by the C oracle's own decoder."""
        b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_decode_array(b.size, b.ctypes.data, out.ctypes.data)
        return out

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns: the upper half of a binary32 word.
    This is the decoder every tolerance comparison of GPU results uses."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):       # signalling NaN patterns widen to quiet NaNs
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


_default: Oracle | None = None


def _stale(library: str = LIBRARY, source: str = SOURCE) -> bool:
    """True when no library exists or the source was changed after it was built."""
    return not os.path.exists(library) or os.path.getmtime(source) > os.path.getmtime(library)


def load(path: str | None = None) -> Oracle:
    """Load the built oracle.  The default library is (re)built first when it
    is missing or older than ``oracle_gemm.c``, so a stale build of an edited
    source is never used."""
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        if _stale():
            build()
        _default = Oracle(LIBRARY)
    return _default
