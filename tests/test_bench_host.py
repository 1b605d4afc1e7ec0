"""Host-side logic of bench.py that needs no GPU: kernel-name parsing for the
traffic summary, the traffic guard against a changed kernel source, and the
one-GPU rule."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cfg_fields():
    assert bench.cfg_fields("Cfg<256, 256, 64, 2, 2, 4, 0, true, 0, false, 16>") == ("barrier", 2)
    assert bench.cfg_fields("Cfg<256, 256, 32, 4, 2, 4, 1, false, 0, false, 32>") == ("flags", 4)
    assert bench.cfg_fields("Cfg<256, 128, 64, 3, 2, 2, 2, true, 4, false, 32>") == ("wavespec", 3)
    # the split-window ring reports the stages value that selects it
    assert bench.cfg_fields("Cfg<256, 256, 64, 2, 2, 4, 0, true, 0, true, 16>") == ("barrier", 5)


def test_mode_runs_cover_every_sync_mode():
    assert set(s for s, _ in bench.MODE_RUNS.values()) == set(bench.SYNC_NAMES.values())
    assert bench.MODE_RUNS["barrier-windows"] == ("barrier", 5)


def test_traffic_only_for_the_profiled_kernel():
    """Traffic is reported only for a workload and (sync mode, stages) that the
    committed summary holds, and only while the kernel source is unchanged."""
    with open(bench.TRAFFIC_FILE) as f:
        info = json.load(f)
    assert info["entries"], "the summary holds at least one kernel configuration"
    for key, e in info["entries"].items():
        assert key == "%s/%d" % (e["sync_mode"], e["stages"])
        got = bench.traffic_per_launch(info["workload"], e["sync_mode"], e["stages"])
        if info["kernel_source_sha256"] == bench.kernel_sha():
            assert got == e["hbm_bytes_per_launch"] == e["fetch_bytes_per_launch"] + e["write_bytes_per_launch"]
        else:
            assert got is None
        assert bench.traffic_per_launch("gemm4096_kn", e["sync_mode"], e["stages"]) is None
    assert bench.traffic_per_launch(info["workload"], "flags", 3) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_helpers_present():
    """Everything main() calls on the GPU path exists (a CPU run never reaches it)."""
    for name in ("time_mode", "cpu_baseline", "traffic_per_launch", "summarize_traffic",
                 "reference_matmul", "other_workloads", "kernel_sha", "parse"):
        assert callable(getattr(bench, name)), name
    import ast
    import builtins
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    defined = {n.name for n in tree.body if isinstance(n, ast.FunctionDef)}
    for n in ast.walk(tree):
        if isinstance(n, (ast.Import, ast.ImportFrom)):
            defined |= {(a.asname or a.name).split(".")[0] for a in n.names}
        elif isinstance(n, ast.Name) and isinstance(n.ctx, ast.Store):
            defined.add(n.id)
    called = {n.func.id for n in ast.walk(tree) if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
    missing = {c for c in called if c not in defined and not hasattr(builtins, c) and c not in dir(bench)}
    assert not missing, missing


def test_stage_sweep_compares_both_all_wave_schemes_at_2_3_4_stages():
    """The 4096^3 configuration compares barrier and flag synchronisation at
    2, 3 and 4 ring stages; every sweep entry must be a valid (sync, stages)
    pair of the library."""
    sweep = bench.STAGE_SWEEPS["gemm4096_kn"]
    for sync in ("barrier", "flags"):
        assert {st for s, st in sweep if s == sync} >= {2, 3, 4}
    for sync, stages in sweep:
        assert sync in ("barrier", "flags")
        assert stages in (2, 3, 4) or (sync, stages) == ("barrier", 5)
