"""bf16 GEMM for MI355X (gfx950): a persistent, circular-buffered, tiled kernel.

The compute path is the HIP library ``libgemm_bf16.so`` built from ``csrc/``;
``binding`` is a thin ctypes layer over its C ABI.  The binding is imported
lazily so that ``inputs`` can be used without loading the HIP library.
"""
from __future__ import annotations

import importlib

__all__ = ["binding", "inputs", "gemm", "GemmError", "SYNC_MODES"]


def __getattr__(name):
    if name in ("gemm", "GemmError", "SYNC_MODES"):
        return getattr(importlib.import_module(__name__ + ".binding"), name)
    raise AttributeError(name)
