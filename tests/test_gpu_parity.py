"""GPU parity: the HIP GEMM (through the C ABI) against the CPU oracle.

Bar (the method's stated acceptance): |gpu - ref| <= 1e-2 * max(1, |ref|) for
every element, computed in fp64 from the bf16 results.  Where fp32
accumulation is exact (small-integer inputs) the bar is bit equality.  Bit
identity between configurations holds within one split signature: plans that
agree on the MFMA block (plan field mfma_block: 16 x 16 x 32 or 32 x 32 x 16)
and on the k split (k_splits, tail_tiles, tail_splits, with the tile bm x bn)
run the same MFMA chain per output element (k in increasing order, 32 or 16
products per MFMA, chunks summed in chunk order), so their outputs must be
bit-identical to each other and from run to run, whatever the sync mode,
stage count or B layout.  Without any split the tile does not matter, so all
configurations with one MFMA block agree.  Across signatures the products are
grouped differently, and results agree to within rounding.

Small cases span several 256 x 256 tiles and ragged tails and are compared in
full.  The five benchmark workloads run at their full sizes, in every
configuration the benchmark times and in its launch configuration, and are
compared in full with the oracle's whole product; an all-ones case checks the
three largest exactly.  Operands of more than 2 GiB are compared on sampled
rows, which the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from pipelined_tiled_dense_amd import binding as bd
from pipelined_tiled_dense_amd.inputs import WORKLOADS, bits, make_operands, workload_operands

pytestmark = pytest.mark.gpu

MODES = [("barrier", 2), ("barrier", 3), ("barrier", 4), ("barrier", bd.STAGES_WINDOWS),
         ("flags", 2), ("flags", 3), ("flags", 4),
         ("wavespec", 2), ("wavespec", 3), ("wavespec", 4),
         ("pingpong", 2), ("pingpong", 3), ("pingpong", 4)]
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    bd.library()
    bd.gemm_bf16_sync_timeouts(reset=True)
    yield
    assert bd.gemm_bf16_sync_timeouts() == 0, "a ring counter wait timed out"


def run(A, B, bt, sync, stages, out=None):
    print("  gemm M=%d K=%d B=%s bt=%s sync=%s stages=%d" % (A.shape[0], A.shape[1], tuple(B.shape),
                                                          bt, sync, stages), flush=True)
    C = bd.gemm(A, B, b_transposed=bt, sync=sync, stages=stages, out=out)
    torch.cuda.synchronize()
    return bits(C.cpu()).copy()


def block_of(M, N, K, bt, sync, stages):
    return bd.gemm_bf16_plan(M, N, K, bt, stages, bd.SYNC_MODES[sync])["mfma_block"]


def assert_same_bits_per_block(outs, what="modes disagree bitwise"):
    """outs: (key, result) pairs, the key an MFMA block edge or a split
    signature; results with one key agree bit for bit."""
    first = {}
    for blk, got in outs:
        if blk in first:
            np.testing.assert_array_equal(got, first[blk], err_msg="%s (%s)" % (what, blk))
        else:
            first[blk] = got
    return first


def decode(b):
    return oracle.bf16_bits_to_f64(b)


def assert_within_tol(got, ref, what):
    g, r = decode(got), decode(ref)
    err = np.abs(g - r)
    lim = TOL * np.maximum(1.0, np.abs(r))
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError("%s: %d/%d elements outside tolerance; first %s got %r want %r" % (
            what, int(bad.sum()), bad.size, tuple(idx), g[tuple(idx)], r[tuple(idx)]))
    same = float(np.mean(got == ref))
    print("  %s: max abs err %.3g, max rel err %.3g, bit-equal %.4f" % (
        what, err.max() if err.size else 0.0,
        (err / np.maximum(1.0, np.abs(r))).max() if err.size else 0.0, same), flush=True)
    return same


SMALL = [
    (256, 256, 256, None),
    (512, 512, 256, None),
    (300, 264, 200, None),          # ragged in M, N and K
    (777, 520, 1000, None),
    (1, 8, 8, None),
    (33, 8, 16, None),
    (256, 256, 8, None),            # K shorter than one k-step
    (513, 1032, 72, None),
    (640, 384, 512, (520, 400)),    # padded leading dimensions for A and B
]


@pytest.fixture(scope="module")
def small_refs():
    cache = {}

    def get(case, bt):
        key = (case, bt)
        if key not in cache:
            M, N, K, lds = case
            lda, ldb = (lds if lds else (None, None))
            if bt and lds:
                ldb = K + 16
            A, B = make_operands(M, N, K, b_transposed=bt, seed=M * 7 + N * 3 + K, lda=lda, ldb=ldb)
            ref = oracle.load().gemm_bf16(bits(A), bits(B), bt, K=K, N=N)
            cache[key] = (A, B, ref)
        return cache[key]
    return get


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%dx%dx%d%s" % (c[0], c[1], c[2], "_ld" if c[3] else ""))
def test_small_parity_all_modes(case, bt, small_refs):
    A, B, ref = small_refs(case, bt)
    dA, dB = A.cuda(), B.cuda()
    outs = []
    for sync, stages in MODES:
        got = run(dA, dB, bt, sync, stages)
        assert_within_tol(got, ref, "%s/%d" % (sync, stages))
        outs.append((block_of(A.shape[0], B.shape[0] if bt else B.shape[1], A.shape[1], bt, sync, stages), got))
    assert_same_bits_per_block(outs)


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("K", [72, 104, 136, 168, 200], ids=lambda k: "K%d" % k)
def test_many_tiles_per_workgroup(K, bt):
    """More output tiles than workgroups (33 x 17 = 561 tiles of 256 x 256, so
    each persistent workgroup walks 2-3 tiles, ragged in M and N), at k-step
    counts on both sides of the point where the load cursor switches from
    entering each new tile itself to having the next tile's origin computed
    ahead by the compute loop: stages + 1 k-steps for 2 stages of 64 and 3
    for the split-window ring (K = 72, 104, 136, 168, 200 give 2, 2, 3, 3, 4),
    stages + 2 for 3 and 4 stages of 32 (3, 4, 5, 6, 7).  A workgroup's third
    tile is where a stale next-tile origin shows: it then repeats the second
    tile.  The split-window ring also stages each tile's epilogue in a window
    the next tile reloads right after."""
    M, N = 8448 - 40, 4104
    A, B = make_operands(M, N, K, b_transposed=bt, seed=K + (1000 if bt else 0))
    ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)
    dA, dB = A.cuda(), B.cuda()
    outs = []
    for sync, stages in MODES:
        got = run(dA, dB, bt, sync, stages)
        assert_within_tol(got, ref, "%s/%d" % (sync, stages))
        outs.append((block_of(M, N, K, bt, sync, stages), got))
    assert_same_bits_per_block(outs)


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_split_k(bt):
    """Few output tiles and a long k range: the k range is cut into chunks whose
    fp32 partial tiles are summed in chunk order.  1000 x 1032 has 20 tiles of
    256 x 256, so K = 8192 splits into 8 chunks of 1024 (ragged M and N); the
    256 x 128 tiles of the wave-specialised 3-stage ring split it into 4, the
    128 x 128 tiles of ping-pong into 2, or into 4 where each MFMA group has a
    ring of its own (two pipelines per workgroup).  Modes with the same split
    signature (tile, chunks, MFMA block) give the same bits, run after run and
    on any stream; a K with no valid chunking stays unsplit."""
    M, N, K = 1000, 1032, 8192
    for sync, stages in MODES:
        plan = bd.gemm_bf16_plan(M, N, K, bt, stages, bd.SYNC_MODES[sync])
        s = {256: 8, 128: 4}[plan["bn"]] if plan["bm"] == 256 else 2 * plan["pipelines"]
        assert plan["k_splits"] == s, (sync, stages, plan)
        assert plan["workspace_bytes"] == plan["tiles"] * s * plan["bm"] * plan["bn"] * 4
    assert bd.gemm_bf16_plan(M, N, K + 8, bt, 0, 0)["k_splits"] == 1
    A, B = make_operands(M, N, K, b_transposed=bt, seed=4242 + bt)
    ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)
    dA, dB = A.cuda(), B.cuda()
    by_sig = {}
    for sync, stages in MODES:
        sig = split_signature(M, N, K, bt, sync, stages)
        got = run(dA, dB, bt, sync, stages)
        assert_within_tol(got, ref, "split %s/%d" % (sync, stages))
        if sig in by_sig:
            np.testing.assert_array_equal(got, by_sig[sig], err_msg="same split, different bits")
        else:
            by_sig[sig] = got
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        C = bd.gemm(dA, dB, b_transposed=bt)
    side.synchronize()
    np.testing.assert_array_equal(bits(C.cpu()), by_sig[split_signature(M, N, K, bt, "barrier", 0)])


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_split_at_half_the_compute_units(bt):
    """Exactly half as many 256 x 256 tiles as compute units (4096 x 2048, 128
    tiles on 256 CUs) and K = 1024: two chunks of 512 for the 256 x 256 tile
    (the loader/MFMA modes' smaller tiles fill the GPU unsplit).  Compared in
    full with the oracle; modes with the same split signature agree bit for
    bit."""
    M, N, K = 4096, 2048, 1024
    cus = bd.gemm_bf16_plan(8192, 8192, 8192, True, 0, 0)["grid"]
    A, B = make_operands(M, N, K, b_transposed=bt, seed=6060 + bt)
    ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)
    dA, dB = A.cuda(), B.cuda()
    outs = []
    for sync, stages in (("barrier", 2), ("barrier", bd.STAGES_WINDOWS), ("flags", 2), ("wavespec", 3),
                         ("pingpong", 3)):
        plan = bd.gemm_bf16_plan(M, N, K, bt, stages, bd.SYNC_MODES[sync])
        if cus == 256:
            assert plan["k_splits"] == (2 if plan["bn"] == 256 else 1), (sync, stages, plan)
        got = run(dA, dB, bt, sync, stages)
        assert_within_tol(got, ref, "half %s/%d" % (sync, stages))
        outs.append((split_signature(M, N, K, bt, sync, stages), got))
    assert_same_bits_per_block(outs, "same split, different bits")


def test_plans():
    """The launch shape each (sync mode, stages) resolves to: 256 x 256 tiles over
    8 waves for the all-wave modes (64-wide k-steps with 2 stages or the split
    window ring, 32-wide with 3 and 4); for the wave-specialised mode 256 x 256
    over 8 MFMA + 4 loader waves with 2 and 4 stages and 256 x 128 over 4 + 4
    with 3; the LDS never exceeds 160 KiB, and the split-window ring (five
    32 KiB windows, epilogue staged inside one) uses all of it."""
    want = {("barrier", 2): (256, 64, 8, 0), ("barrier", 3): (256, 32, 8, 0), ("barrier", 4): (256, 32, 8, 0),
            ("barrier", bd.STAGES_WINDOWS): (256, 64, 8, 0),
            ("flags", 2): (256, 64, 8, 0), ("flags", 3): (256, 32, 8, 0), ("flags", 4): (256, 32, 8, 0),
            ("wavespec", 2): (256, 64, 8, 4), ("wavespec", 3): (128, 64, 4, 4), ("wavespec", 4): (256, 32, 8, 4),
            ("pingpong", 2): (128, 64, 8, 4), ("pingpong", 3): (128, 64, 8, 4), ("pingpong", 4): (128, 64, 8, 4)}
    for (sync, stages), (bn, bk, mw, pw) in want.items():
        bm = 128 if sync == "pingpong" else 256
        for bt in (False, True):
            pl = bd.gemm_bf16_plan(8192, 8192, 8192, bt, stages, bd.SYNC_MODES[sync])
            assert (pl["bm"], pl["bn"], pl["bk"], pl["mfma_waves"], pl["producer_waves"]) == (bm, bn, bk, mw, pw), \
                (sync, stages, pl)
            assert pl["stages"] == stages and pl["threads"] == 64 * (mw + pw), (sync, stages, pl)
            assert pl["lds_bytes"] <= 160 * 1024, (sync, stages, pl)
    pl = bd.gemm_bf16_plan(8192, 8192, 8192, True, bd.STAGES_WINDOWS, 0)
    assert pl["lds_bytes"] == 5 * 256 * 64 * 2
    assert bd.gemm_bf16_plan(8192, 8192, 8192, True, 0, 0)["stages"] == bd.STAGES_WINDOWS
    assert bd.gemm_bf16_plan(8192, 8192, 8192, True, 0, 2)["stages"] == 2
    assert bd.gemm_bf16_plan(8192, 8192, 8192, True, 0, 3)["stages"] == 3
    assert bd.gemm_bf16_plan(8192, 8192, 8192, True, 0, 3)["tiles"] == 64 * 64


def expected_tail(tiles, K, cus):
    """The split-tail rule: a last round of at most half the compute units
    that a k split of s chunks (s <= cus / r, 64 * s | K, K / s >= 1024,
    K - K / s >= 2048) can spread."""
    if tiles <= cus or tiles % cus == 0 or 2 * (tiles % cus) > cus:
        return 0, 0
    r = tiles % cus
    for s in range(min(cus // r, 16), 1, -1):
        if K % (64 * s) == 0 and K // s >= 1024 and K - K // s >= 2048:
            return r, s
    return 0, 0


def test_split_tail_plans():
    """4352 x 4352 x 4096: 289 tiles of 256 x 256 are one full round of the 256
    compute units plus 33, so the last 33 tiles of the schedule run split into
    4 chunks of 1024.  In 256 x 128 tiles: 578 = 512 + 66 -> 3 would leave
    chunks that are no multiple of 64, so 2 chunks; in 128 x 128 tiles:
    1156 = 1024 + 132, more than half a round -> no tail.  Whole rounds
    (8192^3), chunks shorter than 1024, a split that takes less than 2048 off
    the k range (K = 2048) and a K with no valid chunking have none."""
    cus = bd.gemm_bf16_plan(8192, 8192, 8192, True, 0, 0)["grid"]
    for sync, stages in MODES:
        for bt in (False, True):
            pl = bd.gemm_bf16_plan(4352, 4352, 4096, bt, stages, bd.SYNC_MODES[sync])
            r, sp = expected_tail(pl["tiles"], 4096, cus)
            assert (pl["tail_tiles"], pl["tail_splits"]) == (r, sp), (sync, stages, pl)
            assert pl["k_splits"] == 1 and pl["grid"] == min(pl["tiles"] - r, cus), (sync, stages, pl)
            assert pl["workspace_bytes"] == r * sp * pl["bm"] * pl["bn"] * 4, (sync, stages, pl)
            pl = bd.gemm_bf16_plan(8192, 8192, 8192, bt, stages, bd.SYNC_MODES[sync])
            assert (pl["tail_tiles"], pl["tail_splits"], pl["workspace_bytes"]) == (0, 0, 0), (sync, stages, pl)
    if cus == 256:
        pl = bd.gemm_bf16_plan(4352, 4352, 4096, True, 2, 0)
        assert (pl["tail_tiles"], pl["tail_splits"]) == (33, 4)
        assert bd.gemm_bf16_plan(4352, 4352, 4096, True, 3, 2)["tail_splits"] == 2
        assert bd.gemm_bf16_plan(4352, 4352, 4096, True, 3, 3)["tail_tiles"] == 0
        assert bd.gemm_bf16_plan(4352, 4352, 1536, True, 2, 0)["tail_tiles"] == 0
        assert bd.gemm_bf16_plan(4352, 4352, 2048, True, 2, 0)["tail_tiles"] == 0
    assert bd.gemm_bf16_plan(4352, 4352, 4104, True, 2, 0)["tail_tiles"] == 0
    for sync, stages in MODES:   # the device's plan is the host-only plan for its compute units
        for shape in ((4352, 4352, 4096), (1000, 1032, 8192), (300, 264, 200)):
            assert bd.gemm_bf16_plan(*shape, True, stages, bd.SYNC_MODES[sync]) == \
                bd.gemm_bf16_plan_cus(*shape, True, stages, bd.SYNC_MODES[sync], cus), (sync, stages, shape)


def split_signature(M, N, K, bt, sync, stages):
    pl = bd.gemm_bf16_plan(M, N, K, bt, stages, bd.SYNC_MODES[sync])
    return (pl["bm"], pl["bn"], pl["k_splits"], pl["tail_tiles"], pl["tail_splits"], pl["mfma_block"])


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_split_tail(bt):
    """A split tail on a ragged shape: 4300 x 4344 has 17 x 17 tiles of
    256 x 256 (the last tile row and column partial), K = 4096.  Sampled rows
    cover tile rows 12 and 16, i.e. tiles of the main launch and of the tail,
    and both ragged edges.  Modes whose plans split alike agree bit for bit,
    run after run."""
    M, N, K = 4300, 4344, 4096
    A, B = make_operands(M, N, K, b_transposed=bt, seed=5151 + bt)
    rows = np.array([0, 255, 3072, 3101, 3327, 3328, 4095, 4096, 4150, 4299], dtype=np.int64)
    Ab, Bb = bits(A), bits(B)
    ref = oracle.load().gemm_bf16(np.ascontiguousarray(Ab[rows]), Bb, bt)
    dA, dB = A.cuda(), B.cuda()
    by_sig = {}
    tails = 0
    for sync, stages in MODES:
        sig = split_signature(M, N, K, bt, sync, stages)
        tails += sig[3] > 0
        got = run(dA, dB, bt, sync, stages)
        assert_within_tol(got[rows], ref, "tail %s/%d %s" % (sync, stages, sig))
        if sig in by_sig:
            np.testing.assert_array_equal(got, by_sig[sig], err_msg="same split, different bits")
        else:
            by_sig[sig] = got
    assert tails > 0
    again = run(dA, dB, bt, "barrier", 2)
    np.testing.assert_array_equal(again, by_sig[split_signature(M, N, K, bt, "barrier", 2)])


def test_split_tail_exact_integer_inputs():
    """Small integers make every fp32 sum exact, so with or without a split
    tail, and whatever the tile, every mode equals the oracle bit for bit."""
    rng = np.random.default_rng(11)
    M, N, K = 4300, 4344, 4096
    Av = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    Bv = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    A = torch.from_numpy(Av).to(torch.bfloat16)
    B = torch.from_numpy(Bv).to(torch.bfloat16)
    rows = np.array([0, 3100, 3327, 3328, 4096, 4299], dtype=np.int64)
    ref = oracle.load().gemm_bf16(np.ascontiguousarray(bits(A)[rows]), bits(B), True)
    dA, dB = A.cuda(), B.cuda()
    for sync, stages in MODES:
        got = run(dA, dB, True, sync, stages)
        np.testing.assert_array_equal(got[rows], ref, err_msg="%s/%d" % (sync, stages))


UNALIGNED = [(37, 45, 33), (300, 263, 1001), (1, 1, 1), (513, 1031, 77), (2, 9, 4100)]
PAD_MODES = [("barrier", 2), ("barrier", bd.STAGES_WINDOWS), ("flags", 2), ("wavespec", 3), ("pingpong", 3)]


def padded(X, rows, cols):
    Y = torch.zeros((rows, cols), dtype=torch.bfloat16)
    Y[:X.shape[0], :X.shape[1]] = X
    return Y


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("shape", UNALIGNED, ids=lambda c: "%dx%dx%d" % c)
def test_unaligned_shapes(shape, bt):
    """N or K not a multiple of 8 (with sentinel-filled row padding): the call
    runs on zero-padded copies.  It matches the oracle, and equals bit for bit
    the direct call on operands padded by hand to multiples of 8."""
    M, N, K = shape
    N8, K8 = -(-N // 8) * 8, -(-K // 8) * 8
    A, B = make_operands(M, N, K, b_transposed=bt, seed=M + 3 * N + 7 * K, lda=K + 5, ldb=(K if bt else N) + 3)
    ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)
    Ap = padded(A, M, K8).cuda()
    Bp = (padded(B, N8, K8) if bt else padded(B, K8, N8)).cuda()
    dA, dB = A.cuda(), B.cuda()
    for sync, stages in PAD_MODES:
        plan = bd.gemm_bf16_plan(M, N, K, bt, stages, bd.SYNC_MODES[sync])
        assert plan["pad_bytes"] > 0
        got = run(dA, dB, bt, sync, stages)
        assert_within_tol(got, ref, "unaligned %s/%d" % (sync, stages))
        direct = run(Ap, Bp, bt, sync, stages)
        np.testing.assert_array_equal(got, direct[:, :N], err_msg="%s/%d" % (sync, stages))


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_unaligned_pointers_and_leading_dimensions(bt):
    """Aligned sizes, but operands at 2- and 4-byte offsets with odd leading
    dimensions (views into sentinel-filled buffers) and an odd-strided C: the
    padded path, bit-identical to the direct call on contiguous copies."""
    M, N, K = 200, 136, 264
    A, B = make_operands(M, N, K, b_transposed=bt, seed=606 + bt)
    ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)

    def offset_view(X, left, extra):
        buf = torch.full((X.shape[0], X.shape[1] + left + extra), 1.0e30, dtype=torch.bfloat16, device="cuda")
        buf[:, left:left + X.shape[1]] = X.cuda()
        return buf[:, left:left + X.shape[1]]

    vA, vB = offset_view(A, 1, 2), offset_view(B, 2, 3)
    assert vA.data_ptr() % 16 == 2 and vB.data_ptr() % 16 == 4 and vA.stride(0) % 8 != 0
    Cbuf = torch.full((M, N + 5), 7.0, dtype=torch.bfloat16, device="cuda")
    out = Cbuf[:, 1:N + 1]
    C = bd.gemm(vA, vB, b_transposed=bt, out=out)
    torch.cuda.synchronize()
    got = bits(C.cpu()).copy()
    assert_within_tol(got, ref, "offset views")
    direct = run(A.cuda(), B.cuda(), bt, "barrier", 2)
    np.testing.assert_array_equal(got, direct)
    # the columns around the view are untouched
    assert (Cbuf[:, 0] == 7.0).all() and (Cbuf[:, N + 1:] == 7.0).all()


def test_unaligned_zero_k():
    """K == 0 with an odd N: C is +0 everywhere, columns outside untouched."""
    Cbuf = torch.full((5, 14), 3.0, dtype=torch.bfloat16, device="cuda")
    out = Cbuf[:, 1:12]
    A = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((0, 11), dtype=torch.bfloat16, device="cuda")
    bd.gemm(A, B, out=out)
    torch.cuda.synchronize()
    assert (bits(out.cpu()) == 0).all()
    assert (Cbuf[:, 0] == 3.0).all() and (Cbuf[:, 12:] == 3.0).all()


def test_concurrent_split_calls_on_two_streams():
    """Split and padded calls take their temporary memory from the blocks the
    library keeps per device.  Calls on two streams, interleaved with no
    synchronisation between them (a split
    k range on one, a split tail and an off-grid shape on the other), must
    each give the bits of the same call run alone."""
    cases = [((1000, 1032, 8192), True), ((4300, 4344, 4096), False), ((37, 45, 4100), True)]
    ops, want = [], []
    for (M, N, K), bt in cases:
        A, B = make_operands(M, N, K, b_transposed=bt, seed=M + N + K)
        dA, dB = A.cuda(), B.cuda()
        ops.append((dA, dB, bt))
        want.append(run(dA, dB, bt, "barrier", 2))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for i, (dA, dB, bt) in enumerate(ops):
            st = streams[(i + rep) % 2]
            with torch.cuda.stream(st):
                outs.append((i, bd.gemm(dA, dB, b_transposed=bt, sync="barrier", stages=2)))
    torch.cuda.synchronize()
    for i, C in outs:
        np.testing.assert_array_equal(bits(C.cpu()), want[i], err_msg="case %d" % i)


def random_shapes(seed, n):
    """Seeded shapes on the fast path's 8-element grid: ragged M, N and K, and
    every other shape few-tiled with a long k range (multiples of 512), which
    the k split takes in some configurations' tiles and not in others."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if i % 2:
            M = int(rng.integers(1, 1200))
            N = 8 * int(rng.integers(1, 150))
            K = 512 * int(rng.integers(1, 9))
        else:
            M = int(rng.integers(1, 1600))
            N = 8 * int(rng.integers(1, 200))
            K = 8 * int(rng.integers(1, 300))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_random_shapes_all_modes(bt):
    """Twenty-four seeded random shapes (some split along k in some tiles, see
    random_shapes), every mode, compared in full with the oracle; modes with
    the same split signature agree bit for bit."""
    splits = set()
    for M, N, K in random_shapes(9000 + bt, 24):
        A, B = make_operands(M, N, K, b_transposed=bt, seed=M + 7 * N + 13 * K)
        ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)
        dA, dB = A.cuda(), B.cuda()
        outs = []
        for sync, stages in MODES:
            sig = split_signature(M, N, K, bt, sync, stages)
            splits.add(sig[2] > 1)
            got = run(dA, dB, bt, sync, stages)
            assert_within_tol(got, ref, "%dx%dx%d %s/%d" % (M, N, K, sync, stages))
            outs.append((sig, got))
        assert_same_bits_per_block(outs, "%dx%dx%d: same split, different bits" % (M, N, K))
    assert splits == {False, True}


def test_layouts_and_modes_bit_identical():
    M, N, K = 520, 776, 392
    A, B = make_operands(M, N, K, b_transposed=False, seed=99)
    dA, dB, dBt = A.cuda(), B.cuda(), B.t().contiguous().cuda()
    ref = oracle.load().gemm_bf16(bits(A), bits(B), False)
    outs = []
    for sync, stages in MODES:
        for bt, b in ((False, dB), (True, dBt)):
            got = run(dA, b, bt, sync, stages)
            assert_within_tol(got, ref, "%s/%d bt=%s" % (sync, stages, bt))
            outs.append((block_of(M, N, K, bt, sync, stages), got))
    first = assert_same_bits_per_block(outs, "layouts or modes disagree bitwise")
    for sync, stages in (("flags", 3), ("flags", 2)):
        again = run(dA, dB, False, sync, stages)
        np.testing.assert_array_equal(again, first[block_of(M, N, K, False, sync, stages)])


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_exact_integer_inputs_bitwise(bt):
    """Small integers: every fp32 partial sum is exact, so GPU == oracle bit for bit
    (this pins tile placement and the epilogue's rounding)."""
    rng = np.random.default_rng(7)
    M, N, K = 600, 520, 1016
    Av = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    Bv = rng.integers(-4, 5, size=(N, K) if bt else (K, N)).astype(np.float32)
    A = torch.from_numpy(Av).to(torch.bfloat16)
    B = torch.from_numpy(Bv).to(torch.bfloat16)
    ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)
    for sync, stages in MODES:
        got = run(A.cuda(), B.cuda(), bt, sync, stages)
        np.testing.assert_array_equal(got, ref, err_msg="%s/%d" % (sync, stages))


def test_degenerate_sizes():
    dev = "cuda"
    A = torch.ones((4, 16), dtype=torch.bfloat16, device=dev)
    B = torch.ones((16, 8), dtype=torch.bfloat16, device=dev)
    # M == 0 and N == 0: no-ops
    C = torch.full((0, 8), 7.0, dtype=torch.bfloat16, device=dev)
    bd.gemm(A[:0], B, out=C)
    C = torch.full((4, 0), 7.0, dtype=torch.bfloat16, device=dev)
    bd.gemm(A, B[:, :0], out=C)
    # K == 0: C is set to +0 everywhere
    for sync in ("barrier", "flags", "wavespec", "pingpong"):
        C = torch.full((300, 264), 7.0, dtype=torch.bfloat16, device=dev)
        bd.gemm(A[:0].new_empty((300, 0)), B.new_empty((0, 264)), out=C, sync=sync)
        torch.cuda.synchronize()
        assert np.all(bits(C.cpu()) == 0)
    # C = A * B with K = 8 (a single partial k-step)
    A8, B8 = make_operands(300, 264, 8, b_transposed=False, seed=5)
    ref = oracle.load().gemm_bf16(bits(A8), bits(B8), False)
    got = run(A8.cuda(), B8.cuda(), False, "barrier", 2)
    assert_within_tol(got, ref, "K=8")


def test_output_outside_the_matrix_untouched():
    """Stores past M and N are dropped: a wider, taller C buffer keeps its
    sentinel outside the M x N window."""
    M, N, K = 300, 264, 200
    A, B = make_operands(M, N, K, b_transposed=False, seed=3)
    for sync, stages in MODES:
        buf = torch.full((M + 40, N + 48), 3.0, dtype=torch.bfloat16, device="cuda")
        view = buf[:M, :N]
        bd.gemm(A.cuda(), B.cuda(), out=view, sync=sync, stages=stages)
        torch.cuda.synchronize()
        h = buf.cpu().float()
        assert torch.all(h[M:, :] == 3.0) and torch.all(h[:, N:] == 3.0), (sync, stages)


# --- the five workloads at full size --------------------------------------------
def assert_within_tol_full(got, ref, what, rows_per_chunk=2048):
    """The tolerance check on every element of a large result, a block of rows
    at a time (fp64 decoding of the whole matrix at once would need GBs)."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    worst, bad_total, same = 0.0, 0, 0
    for r0 in range(0, got.shape[0], rows_per_chunk):
        g, r = decode(got[r0:r0 + rows_per_chunk]), decode(ref[r0:r0 + rows_per_chunk])
        scale = np.maximum(1.0, np.abs(r))
        err = np.abs(g - r)
        bad = ~(err <= TOL * scale)                       # NaN counts as a violation
        if bad.any() and bad_total == 0:
            idx = np.argwhere(bad)[0]
            first = (r0 + idx[0], idx[1], g[tuple(idx)], r[tuple(idx)])
        bad_total += int(bad.sum())
        worst = max(worst, float(np.nanmax(err / scale)) if err.size else 0.0)
        same += int(np.count_nonzero(got[r0:r0 + rows_per_chunk] == ref[r0:r0 + rows_per_chunk]))
    if bad_total:
        raise AssertionError("%s: %d/%d elements outside tolerance; first at (%d, %d): got %r want %r"
                             % ((what, bad_total, got.size) + first))
    print("  %s: all %d elements within tolerance, max rel err %.3g, bit-equal %.4f"
          % (what, got.size, worst, same / got.size), flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_full_size(name):
    """Each of the five workloads at its full size, in every (sync mode,
    stages) configuration the benchmark times, in its launch configuration:
    every element against the oracle, which computes the whole product.
    Configurations with the same split signature agree bit for bit."""
    import time

    import bench
    w = WORKLOADS[name]
    A, B = workload_operands(w)
    Ab, Bb = bits(A), bits(B)
    t0 = time.time()
    print("  oracle: %s (%d x %d x %d) in full ..." % (name, w.M, w.N, w.K), flush=True)
    ref = oracle.load().gemm_bf16(Ab, Bb, w.b_transposed)
    print("  oracle: %.1f s on %d threads" % (time.time() - t0, oracle.load().num_threads()), flush=True)
    dA, dB = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    by_sig = {}
    configs = bench.timed_configs(name)
    assert len(configs) == 13
    for sync, stages in configs:
        C.fill_(7.0)
        got = run(dA, dB, w.b_transposed, sync, stages, out=C)
        sig = split_signature(w.M, w.N, w.K, w.b_transposed, sync, stages)
        assert_within_tol_full(got, ref, "%s %s/%d %s" % (name, sync, stages, sig))
        if sig in by_sig:
            np.testing.assert_array_equal(got, by_sig[sig], err_msg="same split, different bits")
        else:
            by_sig[sig] = got
    del dA, dB, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gemm8192_nk", "tall32768x1024_k4096_kn", "longk1024_k32768_kn"])
def test_workload_all_ones_exact(name):
    """A = B = 1 at full size: every element is exactly K (a power of two, exact in
    bf16 and in fp32 accumulation), checked for the whole output in every
    configuration the benchmark times."""
    import bench
    w = WORKLOADS[name]
    A = torch.ones((w.M, w.K), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((w.N, w.K) if w.b_transposed else (w.K, w.N), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    for sync, stages in bench.timed_configs(name):
        C.fill_(7.0)
        bd.gemm(A, B, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
        torch.cuda.synchronize()
        assert torch.all(C == float(w.K)), (name, sync, stages)


def sample_rows(M, n=24, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 255, 256, M // 2, M - 257, M - 256, M - 2, M - 1]
    rows = sorted(set([r for r in fixed if 0 <= r < M] + list(rng.integers(0, M, size=n))))
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("which", ["A_nk", "A_kn", "B_kn"])
def test_operand_over_2gib(which):
    """An operand spanning more than 2^31 bytes: the loads then rebuild their
    buffer resources at every position with a capped byte count instead of
    stepping one resource per tile.  Ragged in M, N and K; compared with the
    oracle on sampled rows (A's sampled rows are copied back from the GPU)."""
    K = 8264
    if which.startswith("A"):
        M, N, bt = 131112, 264, which == "A_nk"
    else:
        M, N, bt = 264, 131112, False
    g = torch.Generator(device="cuda").manual_seed(2024 + len(which) + bt)
    A = (torch.rand(M, K, generator=g, device="cuda") * 2 - 1).to(torch.bfloat16)
    B = (torch.rand(*((N, K) if bt else (K, N)), generator=g, device="cuda") * 2 - 1).to(torch.bfloat16)
    assert max(A.numel(), B.numel()) * 2 > 2 ** 31
    rows = sample_rows(M)
    ref = oracle.load().gemm_bf16(bits(A[torch.from_numpy(rows).cuda()].cpu()), bits(B.cpu()), bt)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    outs = []
    for sync, stages in [("barrier", 2), ("barrier", bd.STAGES_WINDOWS), ("flags", 2), ("wavespec", 3),
                         ("pingpong", 3)]:
        C.fill_(7.0)
        got = run(A, B, bt, sync, stages, out=C)
        assert_within_tol(got[rows], ref, "%s %s/%d (sampled %d rows)" % (which, sync, stages, len(rows)))
        outs.append((split_signature(M, N, K, bt, sync, stages), got))
    assert_same_bits_per_block(outs, "same split, different bits")
    del A, B, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_max_leading_dimensions_with_poisoned_padding(bt):
    """Leading dimensions at the accepted maximum (2^22 elements, so every
    operand spans more than 2 GiB) with everything outside the operands'
    M x K, K x N (or N x K) and M x N windows filled with NaN in A and B and a
    sentinel in C: a load past K or N would put NaN into C, a store past N
    would overwrite the sentinel.  Ragged in M, N and K; all modes."""
    LD = 1 << 22
    M, N, K = 300, 264, 1000 if bt else 264
    A, B = make_operands(M, N, K, b_transposed=bt, seed=77 + bt)
    dA = torch.full((M, LD), float("nan"), dtype=torch.bfloat16, device="cuda")
    dA[:, :K] = A.cuda()
    rows_b, cols_b = (N, K) if bt else (K, N)
    dB = torch.full((rows_b, LD), float("nan"), dtype=torch.bfloat16, device="cuda")
    dB[:, :cols_b] = B.cuda()
    ref = oracle.load().gemm_bf16(bits(A), bits(B), bt)
    Cbuf = torch.empty((M, LD), dtype=torch.bfloat16, device="cuda")
    outs = []
    for sync, stages in MODES:
        Cbuf[:, :N + 4096].fill_(3.0)
        got = run(dA[:, :K], dB[:, :cols_b], bt, sync, stages, out=Cbuf[:, :N])
        assert_within_tol(got, ref, "ld 2^22 %s/%d" % (sync, stages))
        assert bool(torch.all(Cbuf[:, N:N + 4096] == 3.0)), (sync, stages)
        outs.append((split_signature(M, N, K, bt, sync, stages), got))
    assert_same_bits_per_block(outs, "same split, different bits")
    del dA, dB, Cbuf
    torch.cuda.empty_cache()
