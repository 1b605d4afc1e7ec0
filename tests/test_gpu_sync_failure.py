"""Failure handling of the counter-synchronised modes on the GPU, forced from
the host: with a spin limit of one poll, waits on ring counters give up while
the data is merely late, so waves read stages before their loads land and
refill stages that are still being read.  The kernels still run to the end
(every loop is finite; every address comes from loop indices, never from
data), the give-ups are counted, and every output element is either NaN --
its tile may have used data a give-up let through -- or exactly the value of
a normal run.  After the default limit is restored, results are exact again.
Barrier sync has no counter waits and is unaffected."""
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
    bd.gemm_bf16_sync_timeouts(reset=True)
    yield
    bd.gemm_bf16_set_sync_spin_limit(0)
    bd.gemm_bf16_sync_timeouts(reset=True)


def run(dA, dB, bt, sync, stages):
    print("  %s/%d M=%d K=%d bt=%s" % (sync, stages, dA.shape[0], dA.shape[1], bt), flush=True)
    C = bd.gemm(dA, dB, b_transposed=bt, sync=sync, stages=stages)
    torch.cuda.synchronize()
    return bits(C.cpu()).copy()


CASES = [((2048, 2048, 2048), False, "flags", 2), ((2048, 2048, 2048), True, "flags", 3),
         ((2048, 2048, 2048), False, "wavespec", 3), ((2048, 2048, 2048), True, "wavespec", 4),
         ((2048, 2048, 2048), True, "wavespec", 2), ((2048, 2048, 2048), False, "wavespec", 2),
         ((2048, 2048, 2048), False, "pingpong", 3), ((2048, 2048, 2048), True, "pingpong", 2),
         ((2048, 2048, 2048), False, "pingpong", 2), ((1024, 1024, 32768), False, "flags", 2),
         ((1024, 1024, 32768), False, "wavespec", 3)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d_%s_%s%d" % (c[0] + (("nk" if c[1] else "kn"),
                                                                                  c[2], c[3])))
def test_forced_give_ups_are_flagged_with_nan(case):
    (M, N, K), bt, sync, stages = case
    A, B = make_operands(M, N, K, b_transposed=bt, seed=M + K + stages)
    dA, dB = A.cuda(), B.cuda()
    good = run(dA, dB, bt, sync, stages)
    assert not np.isnan(bd_decode(good)).any()
    bd.gemm_bf16_sync_timeouts(reset=True)
    for limit in (1, 10, 20, 40):
        prev = bd.gemm_bf16_set_sync_spin_limit(limit)
        try:
            forced = run(dA, dB, bt, sync, stages)
            timeouts = bd.gemm_bf16_sync_timeouts(reset=True)
        finally:
            bd.gemm_bf16_set_sync_spin_limit(prev)
        nan = np.isnan(bd_decode(forced))
        print("    limit %d: give-ups %d, NaN elements %d of %d" % (limit, timeouts, int(nan.sum()), nan.size),
              flush=True)
        if limit == 1:
            assert timeouts > 0
        if timeouts == 0:
            assert not nan.any()
        # every element is either flagged or exactly what a normal run gives
        ok = nan | (forced == good)
        assert ok.all(), "limit %d: %d unflagged wrong elements" % (limit, int((~ok).sum()))
    # the default limit again: exact
    np.testing.assert_array_equal(run(dA, dB, bt, sync, stages), good)
    assert bd.gemm_bf16_sync_timeouts(reset=True) == 0


def test_barrier_sync_is_unaffected_by_the_spin_limit():
    A, B = make_operands(1024, 1024, 2048, b_transposed=True, seed=5)
    dA, dB = A.cuda(), B.cuda()
    good = run(dA, dB, True, "barrier", 2)
    prev = bd.gemm_bf16_set_sync_spin_limit(1)
    try:
        got = run(dA, dB, True, "barrier", 2)
    finally:
        bd.gemm_bf16_set_sync_spin_limit(prev)
    np.testing.assert_array_equal(got, good)
    assert bd.gemm_bf16_sync_timeouts(reset=True) == 0


def test_spin_limit_setting():
    prev = bd.gemm_bf16_set_sync_spin_limit(1000)
    try:
        assert bd.gemm_bf16_set_sync_spin_limit(0) == 1000       # 0 restores the default
        assert bd.gemm_bf16_set_sync_spin_limit(0) == 1 << 22
        with pytest.raises(bd.GemmError):
            bd.gemm_bf16_set_sync_spin_limit(-1)
    finally:
        bd.gemm_bf16_set_sync_spin_limit(prev if prev != 1000 else 0)


def bd_decode(b):
    """bf16 bit patterns -> float64 via numpy (only NaN-ness is used here)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
