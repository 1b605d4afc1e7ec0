"""Host-side logic of bench.py that needs no GPU: the configuration matrix,
kernel-name parsing and dispatch attribution for the counter summary, the
summary's guard against a changed kernel source, and the one-GPU rule."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_family():
    ns = "void (anonymous namespace)::"
    assert bench.kernel_family(ns + "k_gemm<(anonymous namespace)::Cfg<256, 256, 64, 2, 2, 4, 0, true, 0, "
                                    "false, 16>, true, false>((anonymous namespace)::Params)") == "k_gemm"
    assert bench.kernel_family(ns + "k_gemm_ws<Cfg<256, 128, 64, 3>>(Params)") == "k_gemm_ws"
    assert bench.kernel_family(ns + "k_gemm_pp<Cfg<128>>(Params)") == "k_gemm_pp"
    assert bench.kernel_family(ns + "k_gemm_win<Cfg<256>, true, false>(Params)") == "k_gemm_win"
    assert bench.kernel_family(ns + "k_reduce_splits<Cfg<256>>(Params)") == "k_reduce_splits"
    assert bench.kernel_family("__amd_rocclr_copyBuffer") is None
    assert bench.kernel_family("Custom_Cijk_Alik_Bljk_BBS_BH_MT256x256x64_MI16x16x1") is None


def test_every_configuration_is_timed_on_every_workload():
    """Each sync scheme at 2, 3 and 4 stages, plus the split-window ring
    (barrier sync, stages 5), on every workload; the slowest kernels first."""
    from pipelined_tiled_dense_amd.inputs import WORKLOADS
    want = {(s, st) for s in ("barrier", "flags", "wavespec", "pingpong") for st in (2, 3, 4)} | {("barrier", 5)}
    for name in WORKLOADS:
        got = bench.timed_configs(name)
        assert set(got) == want and len(got) == len(want), name
    assert bench.timed_configs("gemm8192_nk")[0][0] == "pingpong"
    assert bench.timed_configs("gemm8192_nk")[-1] == ("barrier", 2)


def _write_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=cols)
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(cols, r)))


def _synthetic_pass(path, counters):
    """A copy kernel, a small host copy, then two calls of a plain GEMM and one
    split call (GEMM + reduction), with per-instance counter values."""
    ns = "void (anonymous namespace)::"
    disp = [("__amd_rocclr_copyBuffer", 1000), ("__amd_rocclr_copyBuffer", 10),
            (ns + "k_gemm<Cfg<256>, true, false>(Params)", 700_000),
            (ns + "k_gemm<Cfg<256>, true, false>(Params)", 700_000),
            (ns + "k_gemm_ws<Cfg<256>>(Params)", 100_000),
            (ns + "k_reduce_splits<Cfg<256>>(Params)", 10_000)]
    rows = []
    for i, (name, ns_) in enumerate(disp):
        for cname, val in counters(name).items():
            for inst in range(2):                     # values are summed over instances
                rows.append((i + 1, name, cname, val / 2, 1000, 1000 + ns_))
    _write_csv(path, rows)


def test_summarize_counters_end_to_end(tmp_path):
    def sq(name):
        if "copy" in name:
            return {"GRBM_GUI_ACTIVE": 8.0}
        return {"GRBM_GUI_ACTIVE": 8 * 1.7 * 700_000, "SQ_VALU_MFMA_BUSY_CYCLES": 0.8 * 1.7 * 700_000 * 1024,
                "SQ_LDS_IDX_ACTIVE": 1000.0, "SQ_LDS_BANK_CONFLICT": 5.0, "SQ_INSTS_SALU": 3e7}

    def fetch(name):
        return {"FETCH_SIZE": 524288.0 if "copy" in name and "rocclr" in name else 1000.0}

    def write(name):
        return {"WRITE_SIZE": 1048576.0 if "copy" in name else 2000.0}

    _synthetic_pass(tmp_path / "sq.csv", sq)
    _synthetic_pass(tmp_path / "f.csv", fetch)
    _synthetic_pass(tmp_path / "w.csv", write)
    manifest = {"calls": [{"workload": "gemm8192_nk", "config": "barrier/2", "calls": 2, "kernels": ["k_gemm"]},
                          {"workload": "longk1024_k32768_kn", "config": "wavespec/3", "calls": 1,
                           "kernels": ["k_gemm_ws", "k_reduce_splits"]}]}
    (tmp_path / "m.json").write_text(json.dumps(manifest))
    out = tmp_path / "counters.json"
    info = bench.summarize_counters([str(tmp_path / n) for n in ("sq.csv", "f.csv", "w.csv", "m.json")],
                                    out_path=str(out))
    cal = info["calibration"]
    assert cal["fetch_scale"] == pytest.approx(2.0) and cal["write_scale"] == pytest.approx(1.0)
    e = info["entries"]["gemm8192_nk"]["barrier/2"]
    assert e["dispatches"] == 2 and e["clock_ghz"] == pytest.approx(1.7) and e["mfma_busy"] == pytest.approx(0.8)
    assert e["duration_us"] == pytest.approx(700.0)
    assert e["lds_bank_conflict_of_active"] == pytest.approx(0.005)
    assert e["fetch_bytes_per_call"] == round(1000 * 1024 * 2.0)
    assert e["write_bytes_per_call"] == round(2000 * 1024 * 1.0)
    s = info["entries"]["longk1024_k32768_kn"]["wavespec/3"]
    assert s["kernels_per_call"] == ["k_gemm_ws", "k_reduce_splits"]
    assert s["fetch_bytes_per_call"] == round(2 * 1000 * 1024 * 2.0)      # both kernels of the call
    assert bench.counters_for("gemm8192_nk", "barrier/2", path=str(out)) == e
    assert bench.counters_for("gemm8192_nk", "flags/2", path=str(out)) is None
    # taken on another kernel source: not used
    stale = json.loads(out.read_text())
    stale["kernel_source_sha256"] = "0" * 64
    out.write_text(json.dumps(stale))
    assert bench.counters_for("gemm8192_nk", "barrier/2", path=str(out)) is None


def test_summarize_counters_with_l2_pass(tmp_path):
    """The optional fifth CSV (TCC_REQ_sum, TCC_HIT_sum, TCC_MISS_sum) adds
    the GEMM kernel's own L2 requests and miss rate; the reduction of a split
    call is left out."""
    def sq(name):
        return {"GRBM_GUI_ACTIVE": 8.0} if "copy" in name else {"GRBM_GUI_ACTIVE": 8 * 1.7 * 700_000}

    def fetch(name):
        return {"FETCH_SIZE": 524288.0 if "copy" in name and "rocclr" in name else 1000.0}

    def write(name):
        return {"WRITE_SIZE": 1048576.0 if "copy" in name else 2000.0}

    def tcc(name):
        if "k_reduce_splits" in name:
            return {"TCC_REQ_sum": 1e9, "TCC_HIT_sum": 0.0, "TCC_MISS_sum": 1e9}
        return {"TCC_REQ_sum": 6.9e7, "TCC_HIT_sum": 5.5e7, "TCC_MISS_sum": 1.4e7}

    for n, f in (("sq.csv", sq), ("f.csv", fetch), ("w.csv", write), ("t.csv", tcc)):
        _synthetic_pass(tmp_path / n, f)
    manifest = {"calls": [{"workload": "gemm8192_nk", "config": "barrier/2", "calls": 2, "kernels": ["k_gemm"]},
                          {"workload": "longk1024_k32768_kn", "config": "wavespec/3", "calls": 1,
                           "kernels": ["k_gemm_ws", "k_reduce_splits"]}]}
    (tmp_path / "m.json").write_text(json.dumps(manifest))
    paths = [str(tmp_path / n) for n in ("sq.csv", "f.csv", "w.csv", "m.json")]
    info = bench.summarize_counters(paths + [str(tmp_path / "t.csv")], out_path=str(tmp_path / "c.json"))
    for wl, cfg in (("gemm8192_nk", "barrier/2"), ("longk1024_k32768_kn", "wavespec/3")):
        e = info["entries"][wl][cfg]
        assert e["l2_requests"] == pytest.approx(6.9e7) and e["l2_misses"] == pytest.approx(1.4e7)
        assert e["l2_miss_rate"] == pytest.approx(1.4 / 6.9, abs=1e-4)
    without = bench.summarize_counters(paths, out_path=str(tmp_path / "c4.json"))
    assert "l2_requests" not in without["entries"]["gemm8192_nk"]["barrier/2"]
    with pytest.raises(SystemExit):
        bench.summarize_counters(paths[:3], out_path=str(tmp_path / "c3.json"))


def test_dispatches_that_do_not_match_the_manifest_are_rejected(tmp_path):
    _synthetic_pass(tmp_path / "sq.csv", lambda name: {"GRBM_GUI_ACTIVE": 1.0})
    wrong = {"calls": [{"workload": "x", "config": "barrier/2", "calls": 3, "kernels": ["k_gemm"]}]}
    with pytest.raises(SystemExit):
        bench._assign(bench._dispatches(tmp_path / "sq.csv"), wrong)
    short = {"calls": [{"workload": "x", "config": "barrier/2", "calls": 1, "kernels": ["k_gemm"]}]}
    with pytest.raises(SystemExit):
        bench._assign(bench._dispatches(tmp_path / "sq.csv"), short)


def test_committed_counters_match_their_source_or_are_ignored():
    if not os.path.exists(bench.COUNTERS_FILE):
        pytest.skip("no committed counter summary")
    info = json.load(open(bench.COUNTERS_FILE))
    for wl, cfgs in info["entries"].items():
        for cfg, e in cfgs.items():
            got = bench.counters_for(wl, cfg)
            assert got == (e if info["kernel_source_sha256"] == bench.kernel_sha() else None)
            assert e["hbm_bytes_per_call"] == e["fetch_bytes_per_call"] + e["write_bytes_per_call"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_helpers_present():
    """Everything main() calls on the GPU path exists (a CPU run never reaches it)."""
    for name in ("time_mode", "measure_workload", "cpu_baseline", "counters_for", "summarize_counters",
                 "reference_matmul", "mfma_ceiling", "counter_run", "kernel_sha", "parse", "sustained",
                 "lds_read_bandwidth", "host_cpu"):
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
        elif isinstance(n, (ast.FunctionDef, ast.arg)):
            defined.add(n.name if isinstance(n, ast.FunctionDef) else n.arg)
    called = {n.func.id for n in ast.walk(tree) if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
    missing = {c for c in called if c not in defined and not hasattr(builtins, c) and c not in dir(bench)}
    assert not missing, missing


def test_summarize_trace_end_to_end(tmp_path):
    """Dispatches of the headline workload's kernels are matched to their
    configuration by name; the table carries the run's events and clocks."""
    ns = "void (anonymous namespace)::"
    k2 = ns + "k_gemm<(anonymous namespace)::Cfg<256, 256, 64, 2, 2, 4, 0, true, 0, false, 16>, true, false>(P)"
    kw = ns + "k_gemm_ws<(anonymous namespace)::Cfg<256, 128, 64, 3, 2, 2, 2, true, 4, false, 16> >(P)"
    kn = ns + "k_gemm<(anonymous namespace)::Cfg<256, 256, 64, 2, 2, 4, 0, false, 0, false, 16>, true, false>(P)"
    rows = [(k2, 700_000), (k2, 710_000), (kw, 900_000), (kn, 5_000)]
    with open(tmp_path / "kt.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        for name, dur in rows:
            wr.writerow({"Kernel_Name": name, "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur})
    line = {"steps": 20, "warmup": 5, "value": 1500.0,
            "roofline": {"kernel": "k_gemm (barrier/2)", "achieved": 1510.0, "frac": 0.6},
            "modes": {"barrier/2": {"kernel_ms_mean": 0.705, "tflops": 1510.0, "clock_ghz": 1.72, "mfma_busy": 0.84},
                      "wavespec/3": {"kernel_ms_mean": 0.9, "tflops": 1200.0}}}
    (tmp_path / "b.json").write_text("# noise\n" + json.dumps(line) + "\n")
    out = bench.summarize_trace(str(tmp_path / "kt.csv"), str(tmp_path / "b.json"), out_path=str(tmp_path / "t.md"))
    text = open(out).read()
    table = [r for r in text.splitlines() if r.startswith("| barrier/2") or r.startswith("| wavespec/3")]
    assert len(table) == 2                                   # the K x N kernel belongs to no headline config
    assert "| 2 | 705.0 | 700.0 | 705.0 | 1510.0 | 1.72 | 0.84 |" in table[0]
    assert "| 1 | 900.0 | 900.0 | 900.0 | 1200.0 | - | - |" in table[1]
    assert "%d clock-sampled calls" % bench.CLOCK_SAMPLE_CALLS in text


def test_sampled_clock_turns_sampling_on_only_for_its_calls():
    """sampled_clock resets the sums, samples exactly its calls with sampling on,
    and restores the previous setting even when a call raises."""
    class FakeBinding:
        def __init__(self, fail_at=None):
            self.on, self.log, self.calls, self.fail_at = False, [], 0, fail_at

        def gemm_bf16_set_clock_sampling(self, enable):
            prev, self.on = self.on, bool(enable)
            self.log.append(("set", bool(enable)))
            return prev

        def gemm_bf16_clock_samples(self, reset=False):
            self.log.append(("read", reset, self.on))
            return {"clock_ghz": 1.75 if self.calls else None}

        def gemm(self, *a, **k):
            self.calls += 1
            self.log.append(("call", self.on))
            if self.fail_at == self.calls:
                raise RuntimeError("launch failed")

    class W:
        b_transposed = True

    fb = FakeBinding()
    assert bench.sampled_clock(fb, None, None, None, W, "barrier", 2, calls=3) == 1.75
    assert fb.log[0] == ("read", True, False)                      # stale sums cleared first
    assert [e for e in fb.log if e[0] == "call"] == [("call", True)] * 3
    assert fb.log[-1] == ("set", False) and fb.on is False         # previous setting restored
    fb = FakeBinding(fail_at=2)
    with pytest.raises(RuntimeError):
        bench.sampled_clock(fb, None, None, None, W, "barrier", 2, calls=3)
    assert fb.on is False


def test_sustained_runs_whole_batches_until_the_time_is_up():
    """bench.sustained with a stand-in GPU: every batch takes 50 ms of event
    time, so 0.12 s needs three batches; the rate is FLOPs over event time."""
    from types import SimpleNamespace

    class Event:
        def __init__(self, enable_timing=False):
            self.t = None

        def record(self):
            fake.clock += 0.0

        def synchronize(self):
            pass

        def elapsed_time(self, other):
            return 50.0

    fake = SimpleNamespace(clock=0.0, calls=0)
    torch_stub = SimpleNamespace(cuda=SimpleNamespace(Event=Event))

    def gemm(A, B, *, b_transposed, sync, stages, out):
        fake.calls += 1

    bd = SimpleNamespace(gemm=gemm)
    w = SimpleNamespace(M=1024, N=1024, K=1024, b_transposed=True)
    r = bench.sustained(bd, w, "barrier", 2, None, None, None, 0.12, torch_stub, batch=10)
    assert fake.calls == 30 and r["calls"] == 30 and r["seconds"] == pytest.approx(0.15)
    flops = 2.0 * 1024 ** 3 * 30
    assert r["tflops"] == pytest.approx(round(flops / 150.0 / 1e9, 2))
    assert r["batch_tflops_min"] == r["batch_tflops_max"] and r["config"] == "barrier/2"


def test_host_cpu_reports_model_and_allowed_cores():
    h = bench.host_cpu()
    assert set(h) == {"model", "cores_allowed"}
    assert h["cores_allowed"] is None or h["cores_allowed"] >= 1
