"""Pins of the gfx950 instruction behaviours the GEMM kernels rely on.

Each test launches one probe wave from ``libgemm_probes.so`` and compares
what the hardware produced with the layout the kernels assume.  Expected
values are built on the CPU from that assumed layout."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "pipelined_tiled_dense_amd", "libgemm_probes.so")


@pytest.fixture(scope="module")
def probes():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    if not os.path.exists(LIB):
        pytest.fail("probe library not built: %s" % LIB)
    lib = ctypes.CDLL(LIB)
    p = ctypes.c_void_p
    lib.gemm_probe_lds_dma.argtypes = [p, p, ctypes.c_int, p, p]
    lib.gemm_probe_mfma.argtypes = [p, p, p, p]
    lib.gemm_probe_mfma16.argtypes = [p, p, p, p]
    lib.gemm_probe_ds_read_tr.argtypes = [p, p, p, p]
    lib.gemm_probe_cvt_bf16.argtypes = [p, p, ctypes.c_int64, p]
    lib.gemm_probe_buffer_oob.argtypes = [p, ctypes.c_int, p, p, p, ctypes.c_int, p]
    lib.gemm_probe_buffer_soffset.argtypes = [p, ctypes.c_int, p, ctypes.c_uint32, p, p]
    for f in (lib.gemm_probe_lds_dma, lib.gemm_probe_mfma, lib.gemm_probe_mfma16, lib.gemm_probe_ds_read_tr,
              lib.gemm_probe_cvt_bf16, lib.gemm_probe_buffer_oob, lib.gemm_probe_buffer_soffset):
        f.restype = ctypes.c_int
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("base", [0, 512, 6144])
def test_lds_dma_lane_layout(probes, base):
    """global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + offset +
    16*l, whatever global chunk the lane fetched; vmcnt(0) covers the write."""
    print("probe lds_dma base=%d" % base, flush=True)
    rng = np.random.default_rng(base)
    src = np.arange(128 * 4, dtype=np.uint32) + 0x10000
    perm = rng.permutation(64).astype(np.int32)
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    d_perm = torch.from_numpy(perm).cuda()
    d_dump = torch.zeros(2048, dtype=torch.int32, device="cuda")
    rc = probes.gemm_probe_lds_dma(d_src.data_ptr(), d_perm.data_ptr(), base, d_dump.data_ptr(),
                                   _stream())
    assert rc == 0
    torch.cuda.synchronize()
    dump = d_dump.cpu().numpy().view(np.uint32)
    want = np.full(2048, 0xDEADBEEF, dtype=np.uint32)
    for l in range(64):
        w0 = (base + 16 * l) // 4
        want[w0:w0 + 4] = src[4 * perm[l]:4 * perm[l] + 4]
        w1 = (base + 1024 + 16 * l) // 4
        want[w1:w1 + 4] = src[4 * (64 + perm[l]):4 * (64 + perm[l]) + 4]
    bad = np.flatnonzero(dump != want)
    assert bad.size == 0, "%d words differ; first at word %d: got %#x want %#x" % (
        bad.size, bad[0], dump[bad[0]], want[bad[0]])


def test_buffer_load_lds_and_store_range_check(probes):
    """Raw buffer loads into LDS write zeros for lanes whose 16 bytes lie past
    the resource's byte count, and raw buffer stores past it are dropped.
    The kernels use this to zero the K tail and to mask ragged C edges."""
    print("probe buffer_oob", flush=True)
    nbytes = 64 * 1024 + 16
    src = (np.arange(nbytes // 4, dtype=np.uint32) | 0x40000000)
    nrec_src = 512 * 16           # chunks 0..511 in range
    nrec_dst = 40 * 16
    voff = np.array([16 * (i * 9 % 37) if i < 40 else 16 * (600 + i) for i in range(64)],
                    dtype=np.uint32)
    voff[5] = 16 * 511            # last in-range chunk
    voff[6] = 16 * 512            # first chunk past the end
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    d_voff = torch.from_numpy(voff.view(np.int32)).cuda()
    d_dump = torch.zeros(2048, dtype=torch.int32, device="cuda")
    d_dst = torch.full((nbytes // 4,), 0x11111111, dtype=torch.int32, device="cuda")
    assert probes.gemm_probe_buffer_oob(d_src.data_ptr(), nrec_src, d_voff.data_ptr(),
                                        d_dump.data_ptr(), d_dst.data_ptr(), nrec_dst,
                                        _stream()) == 0
    torch.cuda.synchronize()
    dump = d_dump.cpu().numpy().view(np.uint32)
    dst = d_dst.cpu().numpy().view(np.uint32)
    want_lds = np.full(2048, 0xDEADBEEF, dtype=np.uint32)
    want_dst = np.full(nbytes // 4, 0x11111111, dtype=np.uint32)
    for l in range(64):
        o = int(voff[l]) & 0xFFF0
        chunk = src[o // 4:o // 4 + 4] if o + 16 <= nrec_src else np.zeros(4, np.uint32)
        want_lds[4 * l:4 * l + 4] = chunk
    for l in range(64):
        o = int(voff[l]) & 0xFFF0
        if o + 16 <= nrec_dst:
            want_dst[o // 4:o // 4 + 4] = want_lds[4 * l:4 * l + 4]
    bad = np.flatnonzero(dump != want_lds)
    assert bad.size == 0, "LDS: %d words differ; first at word %d: got %#x want %#x" % (
        bad.size, bad[0], dump[bad[0]], want_lds[bad[0]])
    bad = np.flatnonzero(dst != want_dst)
    assert bad.size == 0, "dst: %d words differ; first at word %d: got %#x want %#x" % (
        bad.size, bad[0], dst[bad[0]], want_dst[bad[0]])


def test_mfma_32x32x16_bf16_layout(probes):
    """v_mfma_f32_32x32x16_bf16 operand and result layouts:
    A lane l holds A[l%32][8*(l//32) + i], B lane l holds B[8*(l//32) + i][l%32]
    (i = 0..7), and accumulator register r of lane l is
    D[8*(r//4) + 4*(l//32) + r%4][l%32]."""
    print("probe mfma", flush=True)
    rng = np.random.default_rng(1)
    A = rng.integers(-4, 5, size=(32, 16)).astype(np.float32)
    B = rng.integers(-4, 5, size=(16, 32)).astype(np.float32)
    D = A.astype(np.float64) @ B.astype(np.float64)
    a = np.zeros((64, 8), np.float32)
    b = np.zeros((64, 8), np.float32)
    for l in range(64):
        a[l] = A[l % 32, 8 * (l // 32):8 * (l // 32) + 8]
        b[l] = B[8 * (l // 32):8 * (l // 32) + 8, l % 32]
    da = torch.from_numpy(a.reshape(-1)).to(torch.bfloat16).cuda()
    db = torch.from_numpy(b.reshape(-1)).to(torch.bfloat16).cuda()
    dd = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    assert probes.gemm_probe_mfma(da.data_ptr(), db.data_ptr(), dd.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = dd.cpu().numpy().reshape(64, 16)
    want = np.zeros((64, 16))
    for l in range(64):
        for r in range(16):
            want[l, r] = D[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32]
    np.testing.assert_array_equal(got, want)


def test_mfma_16x16x32_bf16_layout(probes):
    """v_mfma_f32_16x16x32_bf16 operand and result layouts:
    A lane l holds A[l%16][8*(l//16) + i], B lane l holds B[8*(l//16) + i][l%16]
    (i = 0..7), and accumulator register r of lane l is D[4*(l//16) + r][l%16]."""
    print("probe mfma16", flush=True)
    rng = np.random.default_rng(2)
    A = rng.integers(-4, 5, size=(16, 32)).astype(np.float32)
    B = rng.integers(-4, 5, size=(32, 16)).astype(np.float32)
    D = A.astype(np.float64) @ B.astype(np.float64)
    a = np.zeros((64, 8), np.float32)
    b = np.zeros((64, 8), np.float32)
    for l in range(64):
        a[l] = A[l % 16, 8 * (l // 16):8 * (l // 16) + 8]
        b[l] = B[8 * (l // 16):8 * (l // 16) + 8, l % 16]
    da = torch.from_numpy(a.reshape(-1)).to(torch.bfloat16).cuda()
    db = torch.from_numpy(b.reshape(-1)).to(torch.bfloat16).cuda()
    dd = torch.zeros(64 * 4, dtype=torch.float32, device="cuda")
    assert probes.gemm_probe_mfma16(da.data_ptr(), db.data_ptr(), dd.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = dd.cpu().numpy().reshape(64, 4)
    want = np.zeros((64, 4))
    for l in range(64):
        for r in range(4):
            want[l, r] = D[4 * (l // 16) + r, l % 16]
    np.testing.assert_array_equal(got, want)


def test_ds_read_b64_tr_b16_layout(probes):
    """ds_read_b64_tr_b16 within each group of 16 lanes: lane 4r+j of the
    group addresses row r, columns 4j..4j+3 of a 4 x 16 block of 16-bit
    elements; lane i of the group receives column i, rows 0..3."""
    print("probe ds_read_tr", flush=True)
    image = np.arange(4096, dtype=np.uint16)
    addr = np.zeros(64, np.uint32)
    want = np.zeros((64, 4), np.uint16)
    row_bytes = 128
    for l in range(64):
        g, i = divmod(l, 16)
        r, j = divmod(i, 4)
        addr[l] = g * 1024 + r * row_bytes + j * 8
    for l in range(64):
        g, i = divmod(l, 16)
        for t in range(4):
            want[l, t] = image[(g * 1024 + t * row_bytes) // 2 + i]
    d_img = torch.from_numpy(image.view(np.int16)).cuda()
    d_addr = torch.from_numpy(addr.view(np.int32)).cuda()
    d_out = torch.zeros(256, dtype=torch.int16, device="cuda")
    assert probes.gemm_probe_ds_read_tr(d_img.data_ptr(), d_addr.data_ptr(), d_out.data_ptr(),
                                        _stream()) == 0
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(np.uint16).reshape(64, 4)
    np.testing.assert_array_equal(got, want)


def test_cvt_bf16_is_round_to_nearest_even(probes):
    """The epilogue's fp32 -> bf16 conversion rounds to nearest, ties to even
    (compared with PyTorch's CPU conversion, which is RNE), on random values,
    exact ties, subnormals, overflow and signed zeros."""
    print("probe cvt", flush=True)
    rng = np.random.default_rng(2)
    with np.errstate(over="ignore"):
        x = (rng.standard_normal(1 << 16) * np.exp2(rng.integers(-130, 128, 1 << 16))).astype(np.float32)
    ties = rng.integers(0, 1 << 16, 4096).astype(np.uint32) << 16 | 0x8000   # exact midpoints
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3961776e38, -3.3961776e38,
                        1e-45, -1e-45, 1.1754942e-38], dtype=np.float32)
    x = np.concatenate([x, ties.view(np.float32), special])
    x = x[np.isfinite(x) | np.isinf(x)]
    if x.size % 2:
        x = x[:-1]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    d_in = torch.from_numpy(x).cuda()
    d_out = torch.zeros(x.size, dtype=torch.int16, device="cuda")
    assert probes.gemm_probe_cvt_bf16(d_in.data_ptr(), d_out.data_ptr(), x.size, _stream()) == 0
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(np.uint16)
    finite = ~np.isnan(x)
    bad = np.flatnonzero(got[finite] != want[finite])
    assert bad.size == 0, "first mismatch x=%r got %#06x want %#06x" % (
        x[finite][bad[0]], got[finite][bad[0]], want[finite][bad[0]])


def test_buffer_range_check_counts_scalar_offset(probes):
    """A raw buffer load with a scalar offset is out of range when vector offset
    plus scalar offset reaches the resource's byte count.  The kernels keep a
    tile's operand resource at the tile origin and move through the k range
    with the scalar offset, so the k-rows of a K x N B tile past K read zeros
    through this check alone."""
    print("probe buffer_soffset", flush=True)
    src = (np.arange(16 * 1024 // 4 + 4, dtype=np.uint32) | 0x20000000)
    nrec, soff = 4096, 1024
    voff = np.zeros(64, dtype=np.uint32)
    voff[:32] = 16 * np.arange(32)                      # below nrec - soff: in range either way
    voff[32:48] = 3072 + 64 * np.arange(16)             # in [nrec - soff, nrec): decides the semantics
    voff[48:] = 4096 + 16 * np.arange(16)               # at or past nrec: out of range either way
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    d_voff = torch.from_numpy(voff.view(np.int32)).cuda()
    d_dump = torch.zeros(2048, dtype=torch.int32, device="cuda")
    assert probes.gemm_probe_buffer_soffset(d_src.data_ptr(), nrec, d_voff.data_ptr(), soff,
                                            d_dump.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = d_dump.cpu().numpy().view(np.uint32)[:256].reshape(64, 4)
    data = np.array([src[(soff + int(v)) // 4:(soff + int(v)) // 4 + 4] for v in voff])
    zero = np.zeros((64, 4), dtype=np.uint32)
    mid = "zeros" if np.array_equal(got[32:48], zero[32:48]) else (
        "data" if np.array_equal(got[32:48], data[32:48]) else "mixed")
    print("  lanes with voff < nrec <= voff + soff read: %s" % mid, flush=True)
    np.testing.assert_array_equal(got[:32], data[:32])
    np.testing.assert_array_equal(got[48:], zero[48:])
    np.testing.assert_array_equal(got[32:48], zero[32:48])


def test_lds_read_bandwidth_is_64_banks_per_clock(probes):
    """The kernels' LDS swizzles and their bank-conflict arithmetic assume 64
    four-byte banks, 256 bytes per clock per compute unit.  Conflict-free
    ds_read_b128 streams from 16 waves of one workgroup per CU, timed with
    each workgroup's own shader-clock stamps, come within 15% of that and
    never above it."""
    print("probe lds_read_bw", flush=True)
    probes.gemm_probe_lds_read_bw.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]
    probes.gemm_probe_lds_read_bw.restype = ctypes.c_int
    blocks, iters = 256, 2048
    sink = torch.empty(blocks * 1024, dtype=torch.int32, device="cuda")
    stamps = torch.zeros((blocks, 2), dtype=torch.int64, device="cuda")
    for _ in range(2):
        assert probes.gemm_probe_lds_read_bw(iters, blocks, sink.data_ptr(), stamps.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    ticks = stamps[:, 0].double().cpu()
    assert bool((ticks > 0).all())
    bpc = (iters + 1) * 128 * 1024 / ticks
    print("  bytes per clock per CU: mean %.1f, min %.1f, max %.1f" % (bpc.mean(), bpc.min(), bpc.max()), flush=True)
    assert float(bpc.mean()) >= 0.85 * 256
    assert float(bpc.max()) <= 256 * 1.01
    assert probes.gemm_probe_lds_read_bw(0, blocks, sink.data_ptr(), None, _stream()) == -1
