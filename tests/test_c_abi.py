"""The C ABI from C: two C99 programs built with gcc against include/ and the
library, with no Python or C++ in between.  plan_from_c.c calls only the
host-side entry points (runs without a GPU) and must agree with the binding;
gemm_from_c.c allocates device memory through the HIP runtime API, calls
gemm_bf16 and gemm_bf16_bt in every sync mode and checks exact results."""
import os
import subprocess

import pytest

from pipelined_tiled_dense_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "pipelined_tiled_dense_amd")
SRC = os.path.join(ROOT, "tests", "c_abi")
ROCM = "/opt/rocm"


def build(tmp_path, name, cflags, libs=()):
    """Compile flags before the source, libraries after it (as-needed linking
    drops a library that comes before its users)."""
    exe = str(tmp_path / name)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include"), *cflags,
           os.path.join(SRC, name + ".c"), "-L", PKG, "-lgemm_bf16", "-Wl,-rpath," + PKG, *libs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return exe


def test_host_entry_points_from_c(tmp_path):
    """Strict C99 (-pedantic -Werror) against the header alone; every plan the
    C program prints equals the binding's, and so does every status text."""
    bd.library()
    exe = build(tmp_path, "plan_from_c", ["-pedantic", "-Werror"])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60, check=True).stdout.splitlines()
    keys = ("bm", "bn", "bk", "stages", "grid", "tiles", "k_splits", "tail_tiles", "tail_splits", "mfma_block",
            "workspace_bytes", "pipelines")
    plans = statuses = 0
    for line in out:
        f = line.split()
        if f[0] == "status":
            assert " ".join(f[2:]) == bd.gemm_bf16_strerror(int(f[1]))
            statuses += 1
            continue
        M, N, K, bt, stages, sync, rc = map(int, f[:7])
        assert rc == bd.GEMM_OK, line
        want = bd.gemm_bf16_plan_cus(M, N, K, bt, stages, sync, 256)
        assert tuple(map(int, f[7:])) == tuple(want[k] for k in keys), line
        plans += 1
    assert plans == 4 * 14 * 2 and statuses == 10


@pytest.mark.gpu
def test_gemm_from_c(tmp_path):
    """Device memory from the HIP runtime API in a C program, every sync mode,
    both B layouts, results exact (small-integer operands)."""
    exe = build(tmp_path, "gemm_from_c", ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")],
                ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    print("  running %s" % exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
