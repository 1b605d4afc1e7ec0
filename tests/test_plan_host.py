"""Host-side planning through the C ABI, without a GPU (gemm_bf16_plan_cus):
the tile configuration per sync mode and stage count, the persistent grid,
the split k range for few-tile shapes, the split tail for a mostly empty last
round, and the workspace they need.  The rules are restated here from their
definitions (the split and tail conditions on K, s and the compute units) and
checked on named shapes and on random ones."""
import ctypes
import random

import pytest

from pipelined_tiled_dense_amd import binding as bd

CUS = 256   # MI355X

MODES = [("barrier", 2), ("barrier", 3), ("barrier", 4), ("barrier", bd.STAGES_WINDOWS),
         ("flags", 2), ("flags", 3), ("flags", 4),
         ("wavespec", 2), ("wavespec", 3), ("wavespec", 4),
         ("pingpong", 2), ("pingpong", 3), ("pingpong", 4)]

# (bm, bn, bk, mfma waves, loader waves) per (sync, stages)
SHAPES = {("barrier", 2): (256, 256, 64, 8, 0), ("barrier", 3): (256, 256, 32, 8, 0),
          ("barrier", 4): (256, 256, 32, 8, 0), ("barrier", bd.STAGES_WINDOWS): (256, 256, 64, 8, 0),
          ("flags", 2): (256, 256, 64, 8, 0), ("flags", 3): (256, 256, 32, 8, 0), ("flags", 4): (256, 256, 32, 8, 0),
          ("wavespec", 2): (256, 256, 64, 8, 4), ("wavespec", 3): (256, 128, 64, 4, 4),
          ("wavespec", 4): (256, 256, 32, 8, 4),
          ("pingpong", 2): (128, 128, 64, 8, 4), ("pingpong", 3): (128, 128, 64, 8, 4),
          ("pingpong", 4): (128, 128, 64, 8, 4)}


# MFMA block edge: 16 x 16 x 32 MFMAs everywhere but the wave-specialised
# 4-stage ring (two MFMA waves per SIMD over 256 x 256 tiles, 32-wide
# stages), whose one fragment set per wave holds 32 x 32 x 16 blocks.  The
# 2-stage ring of that layout reads half a 32-wide k-step of 16 x 16 blocks
# at a time, with either B layout.
def mfma_block(sync, stages, bt):
    if sync == "wavespec" and stages == 4:
        return 32
    return 16


def plan(M, N, K, bt, sync, stages, cus=CUS):
    return bd.gemm_bf16_plan_cus(M, N, K, bt, stages, bd.SYNC_MODES[sync], cus)


def cdiv(a, b):
    return -(-a // b)


# Independent LDS rings per workgroup: the 2-stage ping-pong gives each MFMA
# group its own ring and every other work item.
def pipelines(sync, stages):
    return 2 if (sync, stages) == ("pingpong", 2) else 1


def want_splits(t, K, cus):
    """At most half as many output tiles (in the configuration's tile) as
    pipelines (cus: compute units x pipelines per workgroup): the largest
    s <= 16, s <= cus / tiles, with 64 * s dividing K and K / s >= 512."""
    if t == 0 or 2 * t > cus:
        return 1
    for s in range(min(cus // t, 16), 1, -1):
        if K % (64 * s) == 0 and K // s >= 512:
            return s
    return 1


def want_tail(tiles, K, cus):
    """A last round of r <= cus / 2 tiles: the largest s <= min(16, cus / r)
    with 64 * s dividing K, chunks K / s >= 1024 and K - K / s >= 2048."""
    if tiles <= cus or tiles % cus == 0 or 2 * (tiles % cus) > cus:
        return 0, 0
    r = tiles % cus
    for s in range(min(cus // r, 16), 1, -1):
        if K % (64 * s) == 0 and K // s >= 1024 and K - K // s >= 2048:
            return r, s
    return 0, 0


@pytest.mark.parametrize("sync,stages", MODES)
@pytest.mark.parametrize("bt", [0, 1])
def test_tile_configuration(sync, stages, bt):
    pl = plan(8192, 8192, 8192, bt, sync, stages)
    bm, bn, bk, mw, pw = SHAPES[(sync, stages)]
    assert (pl["bm"], pl["bn"], pl["bk"], pl["mfma_waves"], pl["producer_waves"]) == (bm, bn, bk, mw, pw)
    assert pl["stages"] == stages and pl["sync_mode"] == bd.SYNC_MODES[sync] and pl["b_transposed"] == bt
    assert pl["threads"] == 64 * (mw + pw)
    assert pl["mfma_block"] == mfma_block(sync, stages, bt)
    assert 0 < pl["lds_bytes"] <= 160 * 1024
    assert pl["tiles"] == (8192 // bm) * (8192 // bn)
    assert pl["k_steps"] == 8192 // bk
    assert pl["grid"] == CUS and pl["k_splits"] == 1
    assert (pl["tail_tiles"], pl["tail_splits"], pl["workspace_bytes"]) == (0, 0, 0)


def test_default_stages():
    assert plan(512, 512, 512, 1, "barrier", 0)["stages"] == bd.STAGES_WINDOWS
    assert plan(512, 512, 512, 1, "flags", 0)["stages"] == 2
    assert plan(512, 512, 512, 1, "wavespec", 0)["stages"] == 2
    assert plan(512, 512, 512, 1, "pingpong", 0)["stages"] == 3
    assert plan(512, 512, 512, 1, "barrier", bd.STAGES_WINDOWS)["lds_bytes"] == 5 * 256 * 64 * 2


def test_benchmark_configurations():
    """The five configurations: 256^3 is one tile; 4096^3 one round of 256
    tiles; 8192^3 four rounds; 1024 x 1024 x 32768 has 16 tiles and splits its
    k range 16 ways; 32768 x 1024 x 4096 has two whole rounds."""
    assert plan(256, 256, 256, 0, "barrier", 2)["tiles"] == 1
    assert plan(256, 256, 256, 0, "barrier", 2)["k_splits"] == 1      # K / 2 < 512
    pl = plan(4096, 4096, 4096, 0, "barrier", 2)
    assert (pl["tiles"], pl["grid"], pl["k_splits"], pl["tail_tiles"]) == (256, 256, 1, 0)
    pl = plan(1024, 1024, 32768, 0, "barrier", 2)
    assert (pl["tiles"], pl["k_splits"], pl["grid"], pl["k_steps"]) == (16, 16, 256, 32)
    assert pl["workspace_bytes"] == 16 * 16 * 256 * 256 * 4
    pl = plan(32768, 1024, 4096, 0, "wavespec", 3)
    assert (pl["tiles"], pl["grid"], pl["tail_tiles"]) == (1024, 256, 0)
    # 64 tiles of 128 x 128: 4 chunks give one work item per workgroup; with a
    # ring per MFMA group, 8 chunks give one per group.
    assert plan(1024, 1024, 32768, 0, "pingpong", 3)["k_splits"] == 4
    pl = plan(1024, 1024, 32768, 0, "pingpong", 2)
    assert (pl["tiles"], pl["k_splits"], pl["grid"], pl["k_steps"], pl["pipelines"]) == (64, 8, 256, 64, 2)


def test_split_k_counts_each_configurations_tiles():
    """The split decision counts the configuration's own tiles and pipelines:
    1000 x 1032 is 20 tiles of 256 x 256 (8 chunks of 1024), 36 of 256 x 128
    (4 chunks) and 72 of 128 x 128 (2 chunks; 4 with two pipelines per
    workgroup, 512 / 72 = 7 and 6 and 5 do not divide 8192 in 64s); a K with
    no chunking of 64s stays unsplit."""
    want = {(256, 256, 1): 8, (256, 128, 1): 4, (128, 128, 1): 2, (128, 128, 2): 4}
    for sync, stages in MODES:
        pl = plan(1000, 1032, 8192, 1, sync, stages)
        assert pl["pipelines"] == pipelines(sync, stages), (sync, stages, pl)
        s = want[(pl["bm"], pl["bn"], pl["pipelines"])]
        assert pl["k_splits"] == s == want_splits(pl["tiles"], 8192, CUS * pl["pipelines"]), (sync, stages)
        assert pl["workspace_bytes"] == pl["tiles"] * s * pl["bm"] * pl["bn"] * 4
        assert pl["k_steps"] == 8192 // s // pl["bk"]
        assert plan(1000, 1032, 8200, 1, sync, stages)["k_splits"] == 1


def test_split_k_at_exactly_half_the_compute_units():
    """128 tiles of 256 x 256 on 256 compute units (8192 x 1024): two chunks fill
    the GPU; one more tile row or column of tiles and the shape stays unsplit."""
    pl = plan(8192, 1024, 8192, 1, "barrier", 2)
    assert (pl["tiles"], pl["k_splits"], pl["grid"], pl["k_steps"]) == (128, 2, 256, 64)
    assert plan(8192 + 256, 1024, 8192, 1, "barrier", 2)["k_splits"] == 1      # 132 tiles
    assert plan(4096, 2048, 1024, 0, "flags", 2)["k_splits"] == 2              # chunks of 512
    assert plan(4096, 2048, 1000, 0, "flags", 2)["k_splits"] == 1              # no chunking of 64s
    assert plan(8192, 1024, 8192, 1, "wavespec", 3)["k_splits"] == 1          # 256 tiles of 256 x 128


def test_split_tail_named_shapes():
    pl = plan(4352, 4352, 4096, 1, "barrier", 2)
    assert (pl["tiles"], pl["tail_tiles"], pl["tail_splits"], pl["grid"]) == (289, 33, 4, 256)
    assert pl["workspace_bytes"] == 33 * 4 * 256 * 256 * 4
    assert (plan(4352, 4352, 4096, 1, "wavespec", 3)["tail_tiles"],
            plan(4352, 4352, 4096, 1, "wavespec", 3)["tail_splits"]) == (66, 2)
    assert plan(4352, 4352, 4096, 1, "pingpong", 3)["tail_tiles"] == 0       # 132 > 128
    assert plan(4352, 4352, 2048, 1, "barrier", 2)["tail_tiles"] == 0        # takes only 1024 off
    assert plan(4352, 4352, 4104, 1, "barrier", 2)["tail_tiles"] == 0        # no 64-multiple chunks
    pl = plan(9216, 4096, 4096, 1, "barrier", 2)                             # 576 = 2 * 256 + 64
    assert (pl["tail_tiles"], pl["tail_splits"], pl["grid"]) == (64, 4, 256)


def test_compute_unit_count_changes_the_schedule():
    """The same shape on 304 compute units: 289 tiles fit one round, no tail."""
    pl = plan(4352, 4352, 4096, 1, "barrier", 2, cus=304)
    assert (pl["grid"], pl["tail_tiles"], pl["k_splits"]) == (289, 0, 1)
    assert plan(1024, 1024, 32768, 0, "barrier", 2, cus=64)["k_splits"] == 4


def test_random_shapes_follow_the_rules():
    rng = random.Random(1234)
    for _ in range(400):
        M = rng.choice([1, 7, 100, 256, 300, 1000, 2048, 4300, 8192, 20000, 65536])
        N = 8 * rng.randint(1, 2500)
        K = 8 * rng.randint(1, 8192)
        sync, stages = rng.choice(MODES)
        bt = rng.randint(0, 1)
        cus = rng.choice([8, 64, 80, 256, 304])
        pl = plan(M, N, K, bt, sync, stages, cus)
        bm, bn, bk = pl["bm"], pl["bn"], pl["bk"]
        tiles = cdiv(M, bm) * cdiv(N, bn)
        assert pl["tiles"] == tiles
        assert pl["pipelines"] == pipelines(sync, stages)
        s = want_splits(tiles, K, cus * pipelines(sync, stages))
        assert pl["k_splits"] == s, (M, N, K, sync, stages, cus, pl)
        r, ts = want_tail(tiles, K, cus) if s == 1 else (0, 0)
        assert (pl["tail_tiles"], pl["tail_splits"]) == (r, ts), (M, N, K, sync, stages, cus, pl)
        items = (tiles - r) * s
        assert pl["grid"] == min(items, cus) and 1 <= pl["grid"] <= cus
        assert pl["k_steps"] == cdiv(K // s, bk)
        if s > 1:
            assert pl["workspace_bytes"] == items * bm * bn * 4
            assert (K // s) % 64 == 0 and K // s >= 512
        elif r:
            assert pl["workspace_bytes"] == r * ts * bm * bn * 4
            assert (tiles - r) % cus == 0 and r * ts <= cus and 2 * r <= cus
        else:
            assert pl["workspace_bytes"] == 0


def up256(b):
    return (b + 255) // 256 * 256


def want_pad(M, N, K, bt):
    """Zero-padded copies for aligned operands: K off the 8-element grid pads
    A (M x K8) and B; N off the grid pads B (N8 x K8 or K8 x N8) and C
    (M x N8); each part is rounded up to 256 bytes."""
    N8, K8 = -(-N // 8) * 8, -(-K // 8) * 8
    k_off, n_off = K8 != K, N8 != N
    a = M * K8 * 2 if (k_off and K) else 0
    b = N8 * K8 * 2 if ((k_off or n_off) and K) else 0
    c = M * N8 * 2 if n_off else 0
    return up256(a) + up256(b) + up256(c)


def test_padded_plans():
    """N or K that is not a multiple of 8: the plan is that of the problem
    padded to multiples of 8, plus the bytes of the padded copies."""
    for (M, N, K) in ((37, 45, 33), (300, 263, 1001), (1, 1, 1), (4100, 4352, 4095), (5, 7, 0), (64, 60, 64),
                      (64, 64, 60)):
        for bt in (0, 1):
            for sync, stages in MODES:
                pl = plan(M, N, K, bt, sync, stages)
                ref = plan(M, -(-N // 8) * 8, -(-K // 8) * 8, bt, sync, stages)
                assert pl["pad_bytes"] == want_pad(M, N, K, bt) > 0, (M, N, K, bt, pl)
                ref["pad_bytes"] = pl["pad_bytes"]
                assert pl == ref, (M, N, K, bt, sync, stages)
    assert plan(64, 64, 64, 0, "barrier", 2)["pad_bytes"] == 0


def test_errors():
    with pytest.raises(bd.GemmError) as e:
        plan(64, 64, 64, 0, "barrier", 2, cus=0)
    assert e.value.code == bd.GEMM_ERR_INVALID_VALUE
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_plan_cus(64, 64, 64, 0, 7, 0, CUS)
    assert e.value.code == bd.GEMM_ERR_STAGES
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_plan_cus(64, (1 << 22) + 1, 64, 0, 0, 0, CUS)
    assert e.value.code == bd.GEMM_ERR_UNSUPPORTED_SHAPE
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_plan_cus(1 << 31, 64, 64, 0, 0, 0, CUS)
    assert e.value.code == bd.GEMM_ERR_UNSUPPORTED_SHAPE
    with pytest.raises(bd.GemmError) as e:
        bd.gemm_bf16_plan_cus(64, 64, 64, 0, 5, 1, CUS)           # split windows need barrier sync
    assert e.value.code == bd.GEMM_ERR_STAGES
    rc = bd.library().gemm_bf16_plan_cus(64, 64, 64, 0, 0, 0, CUS, ctypes.POINTER(bd.Plan)())
    assert rc == bd.GEMM_ERR_INVALID_VALUE
