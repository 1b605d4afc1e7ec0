"""Seeded synthetic operands for the bf16 GEMM workloads.

This module draws inputs and nothing else: it holds none of the GEMM's
arithmetic, imports neither the HIP binding nor the CPU oracle, and is the one
piece both sides share.  Every operand is produced on the CPU from a seeded
``torch.Generator`` and rounded to bf16 (round-to-nearest-even), so a GPU run
and an oracle run of the same workload see the same bits.

Recipe (one generator per workload, A drawn before B):
  uniform  : torch.rand(shape) * 2 - 1      then .to(bfloat16)
  normal01 : torch.randn(shape) * 0.1       then .to(bfloat16)
The right operand is drawn directly in its storage shape: K x N when B is
row-major, N x K when it is stored transposed.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    b_transposed: bool     # True: B stored N x K (K contiguous)
    dist_a: str            # "uniform" or "normal01"
    dist_b: str
    seed: int
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def compulsory_bytes(self) -> int:
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)


# The five GEMM shapes the method is exercised on.  ``gemm8192_nk`` is the
# throughput workload; the others are correctness and stress cases.
WORKLOADS = {
    w.name: w for w in [
        Workload("gemm256_kn", 256, 256, 256, False, "uniform", "uniform", 1,
                 "single-tile case, 2-stage ring, barrier sync"),
        Workload("gemm4096_kn", 4096, 4096, 4096, False, "uniform", "uniform", 2,
                 "barrier vs full/empty flags at 2, 3 and 4 stages"),
        Workload("gemm8192_nk", 8192, 8192, 8192, True, "uniform", "uniform", 3,
                 "B stored N x K, persistent grid over 256 x 256 tiles"),
        Workload("longk1024_k32768_kn", 1024, 1024, 32768, False, "uniform", "uniform", 4,
                 "many k-steps, few output tiles"),
        Workload("tall32768x1024_k4096_kn", 32768, 1024, 4096, False, "normal01", "uniform", 5,
                 "tall-skinny, wave-specialised producer/consumer"),
    ]
}


def _draw(gen: torch.Generator, shape, dist: str) -> torch.Tensor:
    if dist == "uniform":
        x = torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal01":
        x = torch.randn(shape, generator=gen, dtype=torch.float32) * 0.1
    else:
        raise ValueError("unknown distribution %r" % dist)
    return x.to(torch.bfloat16)


def make_operands(M: int, N: int, K: int, *, b_transposed: bool, seed: int,
                  dist_a: str = "uniform", dist_b: str = "uniform",
                  lda: int | None = None, ldb: int | None = None):
    """Return (A, B) as CPU bf16 tensors.

    A is M x K; B is K x N, or N x K when ``b_transposed``.  With ``lda`` /
    ``ldb`` larger than the logical row length the tensors are views into
    wider row-padded buffers whose padding is filled with a large sentinel
    (bf16 1.0e30), so a kernel that reads past the logical row gives wrong
    answers instead of silently right ones."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    a = _draw(gen, (M, K), dist_a)
    b_shape = (N, K) if b_transposed else (K, N)
    b = _draw(gen, b_shape, dist_b)
    return _pad(a, lda), _pad(b, ldb)


def _pad(x: torch.Tensor, ld: int | None) -> torch.Tensor:
    rows, cols = x.shape
    if ld is None or ld == cols:
        return x.contiguous()
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    buf = torch.full((rows, ld), 1.0e30, dtype=torch.bfloat16)
    buf[:, :cols] = x
    return buf[:, :cols]


def workload_operands(w: Workload):
    return make_operands(w.M, w.N, w.K, b_transposed=w.b_transposed, seed=w.seed,
                         dist_a=w.dist_a, dist_b=w.dist_b)


def bits(x: torch.Tensor):
    """uint16 numpy view of a CPU bf16 tensor's bit patterns (keeps strides)."""
    import numpy as np
    return x.view(torch.int16).numpy().view(np.uint16)
