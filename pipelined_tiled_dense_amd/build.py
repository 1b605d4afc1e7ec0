"""Build the HIP libraries of this package in-tree (gfx950 only).

``build()`` always recompiles.  Loading code elsewhere only calls it when no
library exists yet.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are kept out of the generated code on purpose.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-shared", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE]

LIBRARIES = {
    "libgemm_bf16.so": "csrc/gemm_bf16.hip",
    "libgemm_probes.so": "csrc/probes.hip",
}


def _compile(src: str, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *HIP_FLAGS, src, "-o", tmp]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout)
        raise RuntimeError("hipcc failed for %s" % src)
    os.replace(tmp, out)


def build() -> list[str]:
    built = []
    for lib, src in LIBRARIES.items():
        out = os.path.join(HERE, lib)
        _compile(os.path.join(HERE, src), out)
        built.append(out)
    return built


if __name__ == "__main__":
    for path in build():
        print(path)
