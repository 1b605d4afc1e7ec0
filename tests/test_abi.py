"""The C-ABI libraries load and export what include/*.h declares, and argument
validation rejects bad calls before touching the device (runs without a GPU)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "pipelined_tiled_dense_amd")

from pipelined_tiled_dense_amd import binding as bd  # noqa: E402

HEADER_LIB = {
    "gemm_bf16.h": "libgemm_bf16.so",
}


def declared_functions(header):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(gemm_\w+)\s*\(", text, re.M)))


def exported(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.split()}


def test_every_header_is_mapped():
    headers = sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert headers == sorted(HEADER_LIB)


@pytest.mark.parametrize("header", sorted(HEADER_LIB))
def test_library_exports_declared_symbols(header):
    lib = os.path.join(PKG, HEADER_LIB[header])
    assert os.path.exists(lib), "build the package first"
    names = declared_functions(os.path.join(ROOT, "include", header))
    assert {"gemm_bf16", "gemm_bf16_bt", "gemm_bf16_noalloc", "gemm_bf16_plan", "gemm_bf16_strerror"} <= set(names)
    syms = exported(lib)
    missing = [n for n in names if n not in syms]
    assert not missing, missing
    dll = ctypes.CDLL(lib)
    for n in names:
        getattr(dll, n)


def test_library_has_no_oracle_dependency():
    """The product library neither links nor names the oracle."""
    lib = os.path.join(PKG, "libgemm_bf16.so")
    out = subprocess.run(["ldd", lib], capture_output=True, text=True).stdout
    assert "oracle" not in out
    assert b"oracle_" not in open(lib, "rb").read()


def test_probe_library_exports():
    syms = exported(os.path.join(PKG, "libgemm_probes.so"))
    for n in ("gemm_probe_lds_dma", "gemm_probe_buffer_oob", "gemm_probe_mfma", "gemm_probe_mfma16",
              "gemm_probe_ds_read_tr", "gemm_probe_cvt_bf16", "gemm_probe_buffer_soffset",
              "gemm_probe_mfma_ceiling", "gemm_probe_wall_clock_hz"):
        assert n in syms


def test_workspace_info_rejects_null_pointers():
    """Checked before the device is touched."""
    assert bd.library().gemm_bf16_workspace_info(None, None, None) == bd.GEMM_ERR_INVALID_VALUE


ALIGNED = 1 << 20        # fake, 16-byte aligned addresses: never dereferenced by these cases


def call(fn, M=64, N=64, K=64, A=ALIGNED, lda=64, B=2 * ALIGNED, ldb=64, C=4 * ALIGNED, ldc=64,
         stages=0, sync=0):
    return fn(M, N, K, A, lda, B, ldb, C, ldc, stages, sync, None)


@pytest.mark.parametrize("fn", [bd.gemm_bf16, bd.gemm_bf16_bt, bd.gemm_bf16_noalloc], ids=["kn", "nk", "noalloc"])
def test_validation_errors(fn):
    assert call(fn, sync=4) == bd.GEMM_ERR_SYNC_MODE
    assert call(fn, sync=-1) == bd.GEMM_ERR_SYNC_MODE
    assert call(fn, stages=1) == bd.GEMM_ERR_STAGES
    assert call(fn, stages=6) == bd.GEMM_ERR_STAGES
    # the split-window ring exists for barrier sync only
    assert call(fn, stages=bd.STAGES_WINDOWS, sync=1) == bd.GEMM_ERR_STAGES
    assert call(fn, stages=bd.STAGES_WINDOWS, sync=2) == bd.GEMM_ERR_STAGES
    assert call(fn, stages=bd.STAGES_WINDOWS, sync=3) == bd.GEMM_ERR_STAGES
    assert call(fn, M=-1) == bd.GEMM_ERR_INVALID_VALUE
    assert call(fn, K=-8) == bd.GEMM_ERR_INVALID_VALUE
    assert call(fn, N=(1 << 22) + 8, ldb=(1 << 22) + 8, ldc=(1 << 22) + 8) == bd.GEMM_ERR_UNSUPPORTED_SHAPE
    assert call(fn, K=(1 << 22) + 8, lda=(1 << 22) + 8, ldb=(1 << 22) + 8) == bd.GEMM_ERR_UNSUPPORTED_SHAPE
    assert call(fn, A=0) == bd.GEMM_ERR_INVALID_VALUE
    assert call(fn, B=0) == bd.GEMM_ERR_INVALID_VALUE
    assert call(fn, C=0) == bd.GEMM_ERR_INVALID_VALUE
    assert call(fn, lda=56) == bd.GEMM_ERR_INVALID_VALUE
    assert call(fn, ldb=56) == bd.GEMM_ERR_INVALID_VALUE
    assert call(fn, ldc=56) == bd.GEMM_ERR_INVALID_VALUE
    # bf16 pointers must be 2-byte aligned
    assert call(fn, A=ALIGNED + 1) == bd.GEMM_ERR_MISALIGNED
    assert call(fn, B=2 * ALIGNED + 3) == bd.GEMM_ERR_MISALIGNED
    assert call(fn, C=4 * ALIGNED + 5) == bd.GEMM_ERR_MISALIGNED
    # C overlapping A or B
    assert call(fn, C=ALIGNED + 64) == bd.GEMM_ERR_ALIAS
    assert call(fn, C=2 * ALIGNED) == bd.GEMM_ERR_ALIAS
    # degenerate sizes are no-ops that need no pointers and no device
    assert call(fn, M=0, A=0, C=0) == bd.GEMM_OK
    assert call(fn, N=0, B=0, C=0) == bd.GEMM_OK


@pytest.mark.parametrize("fn", [bd.gemm_bf16, bd.gemm_bf16_bt], ids=["kn", "nk"])
def test_unaligned_calls_pass_validation(fn):
    """N or K not a multiple of 8, leading dimensions not a multiple of 8 or
    above 2^22, and 2-byte aligned pointers are valid calls (they run on
    zero-padded copies): validation lets them through to the device query.
    Only checked where no GPU is visible, since the addresses are fake."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; these calls would launch on fake addresses")
    for kw in ({"N": 60, "ldb": 64, "ldc": 64}, {"K": 60}, {"N": 1, "K": 3}, {"lda": 68}, {"ldc": 68},
               {"A": ALIGNED + 2}, {"C": 4 * ALIGNED + 8}, {"lda": (1 << 22) + 8, "B": 1 << 40, "C": 1 << 41},
               {"M": 3, "N": 5, "K": 7}):
        assert call(fn, **kw) == bd.GEMM_ERR_DEVICE, kw


def test_ld_rules_follow_layout():
    # B stored K x N needs ldb >= N; stored N x K needs ldb >= K
    assert call(bd.gemm_bf16, N=128, K=64, ldb=64, ldc=128) == bd.GEMM_ERR_INVALID_VALUE
    assert call(bd.gemm_bf16_bt, N=64, K=128, lda=128, ldb=64) == bd.GEMM_ERR_INVALID_VALUE


def test_plan_validation():
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_plan(64, 64, 64, 0, 7, 0)
    assert e.value.code == bd.GEMM_ERR_STAGES
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_plan(64, 64, 64, 0, 0, 9)
    assert e.value.code == bd.GEMM_ERR_SYNC_MODE
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_plan(64, (1 << 22) + 8, 64, 0, 0, 0)
    assert e.value.code == bd.GEMM_ERR_UNSUPPORTED_SHAPE


def test_strerror():
    for code in range(-9, 1):
        s = bd.gemm_bf16_strerror(code)
        assert s and s != "unknown status"
    assert bd.gemm_bf16_strerror(-99) == "unknown status"
    assert bd.gemm_bf16_strerror(12345) == "unknown status"


def test_no_gpu_gives_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert call(bd.gemm_bf16) == bd.GEMM_ERR_DEVICE
    assert call(bd.gemm_bf16_noalloc) == bd.GEMM_ERR_DEVICE


def test_noalloc_scratch_limit_is_declared():
    """The allocation-free entry point's scratch size in the header matches
    the binding, and covers the largest split workspace on 256 compute units
    (one 256 x 256 fp32 partial tile per compute unit)."""
    text = open(os.path.join(ROOT, "include", "gemm_bf16.h")).read()
    m = re.search(r"GEMM_NOALLOC_SCRATCH_BYTES\s*=\s*([0-9 *]+)\s*}", text)
    assert m and eval(m.group(1)) == bd.GEMM_NOALLOC_SCRATCH_BYTES
    worst = max(bd.gemm_bf16_plan_cus(M, N, K, bt, st, sy, 256)["workspace_bytes"]
                for (M, N, K) in ((256, 256, 1 << 16), (1024, 1024, 32768), (4352, 4352, 4096), (256, 4096, 1 << 15))
                for bt in (0, 1) for sy in (0, 1, 2, 3) for st in (0, 2, 3, 4))
    assert 0 < worst <= bd.GEMM_NOALLOC_SCRATCH_BYTES == 256 * 256 * 256 * 4


def test_sync_spin_limit_setting_needs_no_device():
    prev = bd.gemm_bf16_set_sync_spin_limit(1000)
    try:
        assert bd.gemm_bf16_set_sync_spin_limit(7) == 1000
        assert bd.gemm_bf16_set_sync_spin_limit(0) == 7           # 0 restores the default
        assert bd.gemm_bf16_set_sync_spin_limit(0) == 1 << 22
        for bad in (-1, 1 << 32):
            with pytest.raises(bd.GemmError) as e:
                bd.gemm_bf16_set_sync_spin_limit(bad)
            assert e.value.code == bd.GEMM_ERR_INVALID_VALUE
    finally:
        bd.gemm_bf16_set_sync_spin_limit(prev if prev != 1000 else 0)


def test_clock_sampling_setting_needs_no_device():
    """The sampling switch is host state; reading the sums needs a device."""
    prev = bd.gemm_bf16_set_clock_sampling(True)
    try:
        assert bd.gemm_bf16_set_clock_sampling(False) is True
        assert bd.gemm_bf16_set_clock_sampling(False) is False
    finally:
        bd.gemm_bf16_set_clock_sampling(prev)
    assert bd.library().gemm_bf16_clock_samples(None, 0) == bd.GEMM_ERR_INVALID_VALUE
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_clock_samples()
    assert e.value.code == bd.GEMM_ERR_DEVICE
