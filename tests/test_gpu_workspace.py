"""Temporary memory of split and padded calls on the GPU: the library keeps
blocks and reuses them, so repeated calls on one stream allocate nothing after
the first, the calling thread never waits for the GPU, results are those of
the same call run alone, a split call captured in a HIP graph gets its memory
inside the graph, and the kept blocks can be released on request."""
import time

import numpy as np
import pytest
import torch

from pipelined_tiled_dense_amd import binding as bd
from pipelined_tiled_dense_amd.inputs import bits, make_operands

pytestmark = pytest.mark.gpu

SPLIT = (1000, 1032, 8192)      # 20 tiles of 256 x 256 -> 8 chunks, 40 MiB of partial tiles
PADDED = (37, 45, 4100)         # N and K off the 8-element grid: padded copies


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    bd.library()
    yield


def operands(shape, bt, seed):
    A, B = make_operands(*shape, b_transposed=bt, seed=seed)
    return A.cuda(), B.cuda()


def test_repeated_calls_on_one_stream_reuse_kept_blocks():
    """30 split calls and 30 padded calls on one stream, no synchronisation in
    between: at most one new block per kind of call, none taken afterwards,
    and every result equal bit for bit to the first."""
    assert bd.gemm_bf16_plan(*SPLIT, True, 2, 0)["k_splits"] > 1
    sA, sB = operands(SPLIT, True, 11)
    pA, pB = operands(PADDED, False, 12)
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    before = bd.gemm_bf16_workspace_info()
    outs = []
    with torch.cuda.stream(st):
        for _ in range(30):
            outs.append(("split", bd.gemm(sA, sB, b_transposed=True, sync="barrier", stages=2)))
            outs.append(("padded", bd.gemm(pA, pB, sync="barrier", stages=2)))
    torch.cuda.synchronize()
    after = bd.gemm_bf16_workspace_info()
    print("  kept blocks before %s, after %s" % (before, after), flush=True)
    assert after["busy"] == 0
    assert after["blocks"] - before["blocks"] <= 2
    first = {}
    for kind, C in outs:
        got = bits(C.cpu())
        if kind in first:
            np.testing.assert_array_equal(got, first[kind], err_msg=kind)
        else:
            first[kind] = got


def test_split_calls_do_not_make_the_caller_wait():
    """Enqueueing 20 split calls of 1024 x 1024 x 32768 (16 chunks, 64 MiB of
    partial tiles each) takes the host a fraction of the GPU time they take:
    no call waits for the GPU.  (A stream-ordered free per call would hold
    the host for the whole GPU time of every call.)"""
    M, N, K = 1024, 1024, 32768
    assert bd.gemm_bf16_plan(M, N, K, False, 2, 0)["k_splits"] > 1
    A, B = operands((M, N, K), False, 13)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        bd.gemm(A, B, out=C)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    t0 = time.perf_counter()
    for _ in range(20):
        bd.gemm(A, B, out=C)
    host = time.perf_counter() - t0
    e1.record(s)
    torch.cuda.synchronize()
    gpu = e0.elapsed_time(e1) * 1e-3
    print("  host %.1f us per call, GPU %.1f us per call" % (host / 20 * 1e6, gpu / 20 * 1e6), flush=True)
    assert host < 0.6 * gpu


def test_calls_on_two_streams_keep_their_results():
    """Split calls of two sizes alternating over two streams with no
    synchronisation: a block last used on the other stream is taken only
    after that use has finished, so every result equals the call run alone."""
    cases = [((1000, 1032, 8192), True, 21), ((512, 520, 16384), False, 22)]
    ops, want = [], []
    for shape, bt, seed in cases:
        dA, dB = operands(shape, bt, seed)
        assert bd.gemm_bf16_plan(*shape, bt, 2, 0)["k_splits"] > 1
        ops.append((dA, dB, bt))
        want.append(bits(bd.gemm(dA, dB, b_transposed=bt).cpu()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(6):
        for i, (dA, dB, bt) in enumerate(ops):
            with torch.cuda.stream(streams[(i + rep) % 2]):
                outs.append((i, bd.gemm(dA, dB, b_transposed=bt)))
    torch.cuda.synchronize()
    for i, C in outs:
        np.testing.assert_array_equal(bits(C.cpu()), want[i], err_msg="case %d" % i)
    assert bd.gemm_bf16_workspace_info()["busy"] == 0


def test_split_call_under_graph_capture():
    """gemm_bf16 (not the allocation-free entry point) captured in a HIP
    graph: its partial tiles are allocated and freed inside the graph.  Each
    of several replays, with eager split calls (which use the kept blocks)
    and synchronisations between them, gives the eager result."""
    M, N, K = SPLIT
    dA, dB = operands(SPLIT, False, 31)
    assert bd.gemm_bf16_plan(M, N, K, False, 2, 0)["k_splits"] > 1
    want = bits(bd.gemm(dA, dB).cpu())
    kept = bd.gemm_bf16_workspace_info()["blocks"]
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rc = bd.gemm_bf16(M, N, K, dA.data_ptr(), dA.stride(0), dB.data_ptr(), dB.stride(0),
                              C.data_ptr(), C.stride(0), 2, 0, side.cuda_stream)
    assert rc == bd.GEMM_OK
    torch.cuda.synchronize()
    assert bd.gemm_bf16_workspace_info()["blocks"] == kept      # nothing kept from the capture
    other = torch.empty_like(C)
    for rep in range(4):
        C.fill_(7.0)
        bd.gemm(dA, dB, out=other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(C.cpu()), want, err_msg="replay %d" % rep)
        np.testing.assert_array_equal(bits(other.cpu()), want, err_msg="eager %d" % rep)


def test_release_workspaces():
    """After a split and a padded call the library keeps blocks; releasing
    them leaves none, and the same calls then allocate again and give the
    same bits."""
    sA, sB = operands(SPLIT, True, 41)
    pA, pB = operands(PADDED, False, 42)
    want = (bits(bd.gemm(sA, sB, b_transposed=True).cpu()), bits(bd.gemm(pA, pB).cpu()))
    assert bd.gemm_bf16_workspace_info()["blocks"] >= 1
    bd.gemm_bf16_release_workspaces()
    info = bd.gemm_bf16_workspace_info()
    assert (info["blocks"], info["bytes"], info["busy"]) == (0, 0, 0), info
    got = (bits(bd.gemm(sA, sB, b_transposed=True).cpu()), bits(bd.gemm(pA, pB).cpu()))
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    assert bd.gemm_bf16_workspace_info()["blocks"] >= 1
