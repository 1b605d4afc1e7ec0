"""In-kernel clock sampling on the GPU: off by default, results bit for bit
the same with it on, one sample per workgroup that has work in every GEMM
launch of a call (the main launch and the split tail's), and a clock in the
range the boards run at."""
import numpy as np
import pytest
import torch

from pipelined_tiled_dense_amd import binding as bd
from pipelined_tiled_dense_amd.inputs import bits, make_operands

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    bd.library()
    prev = bd.gemm_bf16_set_clock_sampling(False)
    bd.gemm_bf16_clock_samples(reset=True)
    yield
    bd.gemm_bf16_set_clock_sampling(prev)
    bd.gemm_bf16_clock_samples(reset=True)


def samples_per_call(M, N, K, bt, stages, sync):
    """Workgroups with work in the call's GEMM launches, from its plan."""
    pl = bd.gemm_bf16_plan(M, N, K, bt, stages, bd.SYNC_MODES[sync])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    main = min(pl["grid"], (pl["tiles"] - pl["tail_tiles"]) * pl["k_splits"])
    tail = min(pl["tail_tiles"] * pl["tail_splits"], cus) if pl["tail_tiles"] else 0
    return main + tail


CASES = [((2048, 2048, 2048), True, "barrier", 2), ((2048, 2048, 2048), True, "barrier", 5),
         ((2048, 2048, 2048), False, "flags", 3), ((2048, 2048, 2048), False, "wavespec", 3),
         ((2048, 2048, 2048), True, "wavespec", 2), ((2048, 2048, 2048), False, "wavespec", 4),
         ((2048, 2048, 2048), True, "pingpong", 4), ((2048, 2048, 2048), False, "pingpong", 2),
         ((4352, 4352, 4096), False, "barrier", 2),
         ((1024, 1024, 32768), False, "wavespec", 3), ((300, 200, 4104), False, "barrier", 2)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d_%s_%s%d" % (c[0] + (("nk" if c[1] else "kn"),
                                                                                  c[2], c[3])))
def test_sampling_counts_and_leaves_results_unchanged(case):
    (M, N, K), bt, sync, stages = case
    print("  %s/%d M=%d N=%d K=%d bt=%s" % (sync, stages, M, N, K, bt), flush=True)
    A, B = make_operands(M, N, K, b_transposed=bt, seed=M + N + K)
    dA, dB = A.cuda(), B.cuda()
    off = bits(bd.gemm(dA, dB, b_transposed=bt, sync=sync, stages=stages).cpu()).copy()
    assert bd.gemm_bf16_clock_samples(reset=True)["samples"] == 0      # off by default
    calls = 3
    bd.gemm_bf16_set_clock_sampling(True)
    try:
        on = [bits(bd.gemm(dA, dB, b_transposed=bt, sync=sync, stages=stages).cpu()).copy() for _ in range(calls)]
        got = bd.gemm_bf16_clock_samples(reset=True)
    finally:
        bd.gemm_bf16_set_clock_sampling(False)
    for c in on:
        np.testing.assert_array_equal(c, off)
    print("    samples %d, clock %.3f GHz" % (got["samples"], got["clock_ghz"]), flush=True)
    assert got["samples"] == calls * samples_per_call(M, N, K, bt, stages, sync)
    assert 1e6 <= got["wall_hz"] <= 1e9
    assert got["wall_ticks"] > 0 and got["shader_ticks"] > got["wall_ticks"]
    assert 0.3 < got["clock_ghz"] < 3.0
    # cleared by the reset
    again = bd.gemm_bf16_clock_samples()
    assert again["samples"] == 0 and again["shader_ticks"] == 0 and again["wall_ticks"] == 0


def test_sampling_off_adds_nothing():
    A, B = make_operands(512, 512, 512, b_transposed=True, seed=3)
    bd.gemm_bf16_clock_samples(reset=True)
    bd.gemm(A.cuda(), B.cuda(), b_transposed=True)
    torch.cuda.synchronize()
    assert bd.gemm_bf16_clock_samples(reset=True)["samples"] == 0
