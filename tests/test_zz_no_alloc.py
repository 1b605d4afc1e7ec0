"""gemm_bf16_noalloc, the allocation-free variant of gemm_bf16, through the C
ABI: on calls that need temporary memory (split k ranges, a split tail,
padded operand copies) it gives exactly gemm_bf16's bits, also on a second,
smaller call after a larger one (the scratch region keeps the previous
call's contents), and it rejects a call whose temporary memory exceeds its
scratch region before enqueuing anything."""
import numpy as np
import pytest
import torch

import oracle
from pipelined_tiled_dense_amd import binding as bd
from pipelined_tiled_dense_amd.inputs import bits, make_operands

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    bd.library()
    bd.gemm_bf16_sync_timeouts(reset=True)
    yield
    assert bd.gemm_bf16_sync_timeouts() == 0, "a ring counter wait timed out"


def call(fn, A, B, C, sync, stages):
    """One call of a K x N entry point on tensors (any leading dimensions)."""
    M, K = A.shape
    N = B.shape[1]
    print("  %s M=%d N=%d K=%d lda=%d sync=%s stages=%d" % (fn.__name__, M, N, K, A.stride(0), sync, stages),
          flush=True)
    return fn(M, N, K, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0), C.data_ptr(), C.stride(0),
              stages, bd.SYNC_MODES[sync], torch.cuda.current_stream().cuda_stream)


def both(A, B, sync, stages):
    """(gemm_bf16's C, gemm_bf16_noalloc's C) as bf16 bit patterns."""
    out = []
    for fn in (bd.gemm_bf16, bd.gemm_bf16_noalloc):
        C = torch.full((A.shape[0], B.shape[1]), 7.0, dtype=torch.bfloat16, device="cuda")
        assert call(fn, A, B, C, sync, stages) == bd.GEMM_OK
        torch.cuda.synchronize()
        out.append(bits(C.cpu()).copy())
    return out


CASES = [
    # (M, N, K, lda pad, what): the first needs all 64 MiB (16 tiles x 16 chunks of 256 x 256 fp32)
    (1024, 1024, 32768, 0, "split k range, whole scratch region"),
    (1000, 1032, 8192, 0, "smaller split k range after a larger one"),
    (4300, 4344, 4096, 0, "split tail"),
    (300, 264, 4096, 3, "padded A copy and a split k range"),
    (37, 45, 33, 0, "N and K off the 8-element grid"),
    (520, 776, 392, 0, "no temporary memory"),
]


@pytest.mark.parametrize("sync,stages", [("barrier", 2), ("barrier", 0), ("wavespec", 0), ("wavespec", 3), ("pingpong", 2),
                                         ("pingpong", 3), ("flags", 2)])
def test_noalloc_equals_gemm_bf16(sync, stages):
    """Every case in order (larger temporary memory first), same bits as
    gemm_bf16; the largest and a padded one also against the oracle."""
    for M, N, K, pad, what in CASES:
        plan = bd.gemm_bf16_plan(M, N, K, False, stages, bd.SYNC_MODES[sync])
        A, B = make_operands(M, N, K, b_transposed=False, seed=M + N + K, lda=K + pad if pad else None)
        dA = torch.full((M, K + pad), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :K] if pad else A.cuda()
        if pad:
            dA.copy_(A.cuda())
        dB = B.cuda()
        ref_call, got = both(dA, dB, sync, stages)
        np.testing.assert_array_equal(got, ref_call, err_msg="%s (%s/%d, plan %s)" % (what, sync, stages, plan))
        if K <= 4096 and M * N <= 1 << 21:
            ref = oracle.load().gemm_bf16(bits(A), bits(B), False)
            g, r = oracle.bf16_bits_to_f64(got), oracle.bf16_bits_to_f64(ref)
            assert np.all(np.abs(g - r) <= TOL * np.maximum(1.0, np.abs(r))), what
        print("    %s: bit-identical (k_splits %d, tail %d, pad %d, workspace %d)" % (
            what, plan["k_splits"], plan["tail_tiles"], plan["pad_bytes"], plan["workspace_bytes"]), flush=True)


def test_noalloc_twice_in_a_row_smaller_second():
    """Two calls in a row on one stream without a synchronisation between
    them, the second smaller: each equals gemm_bf16."""
    A1, B1 = make_operands(1024, 1024, 32768, b_transposed=False, seed=1)
    A2, B2 = make_operands(1000, 1032, 8192, b_transposed=False, seed=2)
    d = [(A1.cuda(), B1.cuda()), (A2.cuda(), B2.cuda())]
    want = [both(a, b, "barrier", 2)[0] for a, b in d]
    outs = []
    for a, b in d:
        C = torch.empty((a.shape[0], b.shape[1]), dtype=torch.bfloat16, device="cuda")
        assert call(bd.gemm_bf16_noalloc, a, b, C, "barrier", 2) == bd.GEMM_OK
        outs.append(C)
    torch.cuda.synchronize()
    for C, w in zip(outs, want):
        np.testing.assert_array_equal(bits(C.cpu()), w)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """An off-grid K needs padded copies of A and B: at 8191^3 they alone are
    about 268 MB, far beyond 64 MiB, so the call returns GEMM_ERR_SCRATCH and
    enqueues nothing (C keeps its contents).  gemm_bf16 runs it."""
    M = N = K = 8191
    A = torch.ones((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((K, N), dtype=torch.bfloat16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    assert bd.gemm_bf16_plan(M, N, K, False, 0, 0)["pad_bytes"] > bd.GEMM_NOALLOC_SCRATCH_BYTES
    assert call(bd.gemm_bf16_noalloc, A, B, C, "barrier", 2) == bd.GEMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(C == 3.0))
    assert "scratch" in bd.gemm_bf16_strerror(bd.GEMM_ERR_SCRATCH)
    assert call(bd.gemm_bf16, A, B, C, "barrier", 2) == bd.GEMM_OK
    torch.cuda.synchronize()
    assert bool(torch.all(C == 8192.0))       # 8191 rounds to 8192 in bf16


def test_noalloc_zero_k():
    """K == 0 writes +0 (a fill kernel, no memset), columns outside untouched."""
    Cbuf = torch.full((5, 14), 3.0, dtype=torch.bfloat16, device="cuda")
    out = Cbuf[:, 1:12]
    A = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    rc = bd.gemm_bf16_noalloc(5, 11, 0, A.data_ptr(), 8, A.data_ptr(), 16, out.data_ptr(), out.stride(0), 0, 0,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == bd.GEMM_OK
    torch.cuda.synchronize()
    assert (bits(out.cpu()) == 0).all()
    assert (Cbuf[:, 0] == 3.0).all() and (Cbuf[:, 12:] == 3.0).all()


def test_noalloc_under_graph_capture():
    """The use gemm_bf16_noalloc exists for: a split call (fp32 partial tiles
    in the scratch region, then the reduction) captured in a HIP graph and
    replayed several times, with eager work and synchronisations between the
    replays, each replay checked against the eager result.  The library is
    used eagerly first, so its one-time device setup happens outside the
    capture."""
    M, N, K = 1000, 1032, 8192
    A, B = make_operands(M, N, K, b_transposed=False, seed=77)
    dA, dB = A.cuda(), B.cuda()
    assert bd.gemm_bf16_plan(M, N, K, False, 2, 0)["k_splits"] > 1
    want = both(dA, dB, "barrier", 2)[0]
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rc = bd.gemm_bf16_noalloc(M, N, K, dA.data_ptr(), dA.stride(0), dB.data_ptr(), dB.stride(0),
                                      C.data_ptr(), C.stride(0), 2, 0, side.cuda_stream)
    assert rc == bd.GEMM_OK
    torch.cuda.synchronize()
    other = torch.empty_like(C)
    for rep in range(4):
        C.fill_(7.0)
        # eager work between replays: another call that uses the same scratch region
        assert call(bd.gemm_bf16_noalloc, dA[:512], dB, other, "barrier", 2) == bd.GEMM_OK
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(C.cpu()), want, err_msg="replay %d" % rep)
