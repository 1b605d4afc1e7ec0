#!/usr/bin/env python3
"""Throughput of the pipelined persistent bf16 GEMM on one MI355X.

A step is one C = A * B over the whole throughput workload (8192 x 8192 x 8192,
B stored N x K, seeded uniform[-1, 1) bf16 inputs already resident in HBM).
Each sync mode (barrier, flags, wave-specialised) is timed at its default
stage count, and barrier sync also over the split-window ring
("barrier-windows"); ``value`` is the fastest and every one is listed under
``modes``.  Prints one JSON line.

Also reports:
  roofline      achieved matrix-core TFLOP/s of the GEMM kernel (2*M*N*K per
                launch / mean launch time from HIP events on the launch
                stream) against the dense bf16 peak, plus HBM traffic per
                launch from the committed rocprofv3 counter summary when it
                matches the current kernel source;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same product
                (a few rows of C), on the host cores it actually uses;
  reference     torch.matmul (hipBLASLt) on the same operands in the same
                process, as context: under the board's power limit the
                attainable clock varies from one GPU to the next.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sync all|barrier|flags|wavespec|barrier-windows]
                       [--stages S] [--workload NAME] [--no-cpu-baseline] [--copy-calibration]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm8192_nk.json")
KERNEL_SOURCE = os.path.join(ROOT, "pipelined_tiled_dense_amd", "csrc", "gemm_bf16.hip")


def kernel_sha():
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sync", default="all",
                    choices=["all", "barrier", "flags", "wavespec", "pingpong", "barrier-windows"])
    ap.add_argument("--stages", type=int, default=0)
    ap.add_argument("--workload", default="gemm8192_nk")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device-to-device copy of known size (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("GEMM_FETCH_CSV", "GEMM_WRITE_CSV",
                                                            "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs into the traffic "
                         "summary read by the roofline line (no GPU needed)")
    ap.add_argument("--traffic-kernel", default="Cfg<256, 256, 64, 2, 2, 4, 0, true, 0, false, 16>",
                    help="kernel configuration the counter CSVs were taken for (a substring of "
                         "the kernel name: Cfg<BM, BN, BK, S, WM, WN, SYNC, B_NxK, loader waves, windows, MFMA block>)")
    ap.add_argument("--no-reference", action="store_true", help="skip the torch.matmul timing")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-workload summary of the other configurations")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def _counter_per_dispatch(path, counter, name_filter):
    """Mean value of `counter` per dispatch of kernels whose name contains
    name_filter, from a rocprofv3 counter_collection CSV (values summed over
    counter instances within a dispatch)."""
    import csv
    per = {}
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter or name_filter not in row["Kernel_Name"]:
            continue
        per[row["Dispatch_Id"]] = per.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit("no %s samples for kernels matching %r in %s" % (counter, name_filter, path))
    return sum(per.values()) / len(per), len(per)


SYNC_NAMES = {0: "barrier", 1: "flags", 2: "wavespec", 3: "pingpong"}
# Timed configurations: label -> (sync mode, stages; 0 = the mode's default).
# "barrier-windows" is barrier sync over the split-window ring.
# They run in this order: the first launches of a process meet a cool chip
# whose clock then settles under the power limit, so the slowest mode (never
# the headline) goes first.
MODE_RUNS = {"pingpong": ("pingpong", 0), "wavespec": ("wavespec", 0), "flags": ("flags", 0),
             "barrier": ("barrier", 0), "barrier-windows": ("barrier", 5)}
# Workloads whose configuration asks for a comparison of the two all-wave
# synchronisation schemes over the ring depth: (sync, stages) runs, reported
# as "sync/stages" -> TFLOP/s (stages 5 is the split-window ring).
STAGE_SWEEPS = {"gemm4096_kn": (("flags", 2), ("flags", 3), ("flags", 4),
                                ("barrier", 2), ("barrier", 3), ("barrier", 4), ("barrier", 5))}


def cfg_fields(kname):
    """(sync mode, stages) of a Cfg<BM, BN, BK, S, WM, WN, SYNC, B_NxK, NP,
    windows, MFMA block> string; the split-window ring reports its stages value, 5."""
    f = [x.strip() for x in kname[kname.index("<") + 1:].rstrip(">").split(",")]
    if len(f) > 9 and f[9] == "true":
        return SYNC_NAMES[int(f[6])], 5
    return SYNC_NAMES[int(f[6])], int(f[3])


def summarize_traffic(paths, kname):
    """FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  Each is scaled by
    the ratio of the known bytes a plain 1 GiB device copy moves to what the
    same counter reads for that copy.  The result is stored in the traffic
    summary under "<sync>/<stages>", next to the entries of other kernel
    configurations profiled on the same kernel source."""
    gf, gw, cf, cw = paths
    sync, stages = cfg_fields(kname)
    fetch_kib, n_f = _counter_per_dispatch(gf, "FETCH_SIZE", kname)
    write_kib, n_w = _counter_per_dispatch(gw, "WRITE_SIZE", kname)
    copy_f_kib, _ = _counter_per_dispatch(cf, "FETCH_SIZE", "copy")
    copy_w_kib, _ = _counter_per_dispatch(cw, "WRITE_SIZE", "copy")
    f_scale = COPY_BYTES / (copy_f_kib * 1024.0)
    w_scale = COPY_BYTES / (copy_w_kib * 1024.0)
    fetch = fetch_kib * 1024.0 * f_scale
    write = write_kib * 1024.0 * w_scale
    try:
        with open(TRAFFIC_FILE) as f:
            out = json.load(f)
        if out.get("kernel_source_sha256") != kernel_sha() or "entries" not in out:
            out = None
    except (OSError, ValueError):
        out = None
    if out is None:
        out = {"workload": "gemm8192_nk", "kernel_source_sha256": kernel_sha(),
               "compulsory_bytes_per_launch": 2 * (3 * 8192 * 8192), "entries": {}}
    out["entries"]["%s/%d" % (sync, stages)] = {
        "kernel": kname,
        "sync_mode": sync,
        "stages": stages,
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch + write),
        "raw_fetch_kib": fetch_kib, "raw_write_kib": write_kib,
        "copy_fetch_kib": copy_f_kib, "copy_write_kib": copy_w_kib,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "dispatches": {"fetch": n_f, "write": n_w},
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def time_mode(bd, dA, dB, C, w, sync, stages, steps, warmup, torch):
    for _ in range(warmup):
        bd.gemm(dA, dB, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        bd.gemm(dA, dB, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, per_launch_ms


def cpu_baseline(w, A, B, target_s):
    import numpy as np

    import oracle
    from pipelined_tiled_dense_amd.inputs import bits
    o = oracle.load()
    Ab, Bb = bits(A), bits(B)
    threads = o.num_threads()
    # calibrate on a few rows, then run a sample sized for ~target_s seconds
    cal_rows = max(1, threads)
    t0 = time.perf_counter()
    o.gemm_bf16(np.ascontiguousarray(Ab[:cal_rows]), Bb, w.b_transposed)
    t_cal = time.perf_counter() - t0
    rows = int(max(cal_rows, min(w.M, cal_rows * target_s / max(t_cal, 1e-6))))
    rows = max(threads, (rows // threads) * threads)
    t0 = time.perf_counter()
    o.gemm_bf16(np.ascontiguousarray(Ab[:rows]), Bb, w.b_transposed)
    t = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "rows 0..%d of C (%d x %d x %d, %.3g GFLOP) in %.2f s; fp64 triple loop, "
                      "one bf16 rounding" % (rows - 1, rows, w.N, w.K, flops / 1e9, t)}


def traffic_per_launch(workload, sync, stages):
    """HBM bytes per launch from the committed counter summary, or None when
    it holds no entry for this kernel configuration or was taken on an older
    kernel source."""
    try:
        info = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if info.get("kernel_source_sha256") != kernel_sha() or info.get("workload") != workload:
        return None
    entry = info.get("entries", {}).get("%s/%d" % (sync, stages))
    return entry.get("hbm_bytes_per_launch") if entry else None


def reference_matmul(dA, dB, C, w, steps, warmup, torch):
    """torch.matmul on the same operands (B^T as a view when B is stored N x K)."""
    Bop = dB.t() if w.b_transposed else dB
    for _ in range(warmup):
        torch.matmul(dA, Bop, out=C)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.matmul(dA, Bop, out=C)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"library": "torch.matmul (hipBLASLt)", "tflops": round(2.0 * w.M * w.N * w.K / ms / 1e9, 2),
            "ms_per_step": round(ms, 4)}


def other_workloads(bd, skip, args, torch):
    """The other configurations, each at every sync mode's default stage count:
    best mode's TFLOP/s (HIP events around all launches) and torch.matmul on
    the same operands."""
    from pipelined_tiled_dense_amd.inputs import WORKLOADS, workload_operands
    out = {}
    for name, w in WORKLOADS.items():
        if name == skip:
            continue
        A, B = workload_operands(w)
        dA, dB = A.cuda(), B.cuda()
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        flops = 2.0 * w.M * w.N * w.K
        per_mode = {}
        for m in ("pingpong", "wavespec", "flags", "barrier"):
            _, per = time_mode(bd, dA, dB, C, w, m, 0, args.steps, args.warmup, torch)
            per_mode[m] = flops / (sum(per) / len(per) * 1e-3) / 1e12
        best = max(per_mode, key=per_mode.get)
        plan = bd.gemm_bf16_plan(w.M, w.N, w.K, w.b_transposed, 0, bd.SYNC_MODES[best])
        entry = {"M": w.M, "N": w.N, "K": w.K, "b_layout": "N x K" if w.b_transposed else "K x N",
                 "best_mode": best, "tflops": round(per_mode[best], 2),
                 "modes_tflops": {m: round(v, 2) for m, v in per_mode.items()},
                 "k_splits": plan["k_splits"]}
        if name in STAGE_SWEEPS:
            sweep = {}
            for sync, stages in STAGE_SWEEPS[name]:
                _, per = time_mode(bd, dA, dB, C, w, sync, stages, args.steps, args.warmup, torch)
                sweep["%s/%d" % (sync, stages)] = round(flops / (sum(per) / len(per) * 1e-3) / 1e12, 2)
            entry["sync_stages_tflops"] = sweep
        if not args.no_reference:
            entry["reference_tflops"] = reference_matmul(dA, dB, C, w, args.steps, args.warmup, torch)["tflops"]
        out[name] = entry
        print("# workload %s: %s" % (name, json.dumps(entry)), file=sys.stderr, flush=True)
        del dA, dB, C
    return out


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.traffic_kernel)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GEMM has no multi-GPU path in this build "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from pipelined_tiled_dense_amd import binding as bd
    from pipelined_tiled_dense_amd.inputs import WORKLOADS, workload_operands

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    bd.library()

    if args.copy_calibration:
        nbytes = COPY_BYTES
        src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes}))
        return

    w = WORKLOADS[args.workload]
    A, B = workload_operands(w)
    dA, dB = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    modes = list(MODE_RUNS) if args.sync == "all" else [args.sync]
    if args.stages != 0 and args.sync == "all":
        modes = ["pingpong", "wavespec", "flags", "barrier"]
    flops = 2.0 * w.M * w.N * w.K
    results = {}
    for m in modes:
        sync, stages = MODE_RUNS[m]
        stages = stages or args.stages
        plan = bd.gemm_bf16_plan(w.M, w.N, w.K, w.b_transposed, stages, bd.SYNC_MODES[sync])
        wall, per = time_mode(bd, dA, dB, C, w, sync, stages, args.steps, args.warmup, torch)
        mean_ms = sum(per) / len(per)
        results[m] = {"sync": sync, "stages": plan["stages"], "tile": "%dx%dx%d" % (plan["bm"], plan["bn"], plan["bk"]),
                      "grid": plan["grid"], "ms_per_step": wall * 1e3 / args.steps,
                      "kernel_ms_mean": mean_ms, "kernel_ms_median": sorted(per)[len(per) // 2],
                      "kernel_ms_min": min(per),
                      "tflops": flops / (wall / args.steps) / 1e12,
                      "kernel_tflops": flops / (mean_ms * 1e-3) / 1e12}
        print("# %s: %s" % (m, json.dumps(results[m])), file=sys.stderr, flush=True)
    timeouts = bd.gemm_bf16_sync_timeouts()
    best = max(results, key=lambda k: results[k]["tflops"])
    r = results[best]
    achieved = r["kernel_tflops"]
    line = {
        "metric": "bf16 GEMM TFLOP/s and % of MFMA peak at 1 GPU (8192^3, per sync mode)",
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "b_layout": "N x K (K contiguous)" if w.b_transposed else "K x N",
                   "inputs": "seeded uniform[-1,1) rounded to bf16, seed %d" % w.seed,
                   "sync_mode": r["sync"], "stages": r["stages"], "tile": r["tile"], "grid": r["grid"],
                   "accumulate": "fp32", "output": "bf16 (RNE)"},
        "pct_of_peak": round(100.0 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
        "modes": {m: {"tflops": round(v["tflops"], 2), "pct_of_peak": round(100 * v["tflops"] / PEAK_BF16_TFLOPS, 2),
                      "stages": v["stages"], "tile": v["tile"], "kernel_ms_mean": round(v["kernel_ms_mean"], 4),
                      "kernel_ms_median": round(v["kernel_ms_median"], 4), "kernel_ms_min": round(v["kernel_ms_min"], 4)}
                  for m, v in results.items()},
        "sync_timeouts": timeouts,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_per_launch(w.name, r["sync"], r["stages"]),
                     "kernel": ("k_gemm_ws (%d stages)" % r["stages"] if r["sync"] == "wavespec"
                                else "k_gemm_pp (%d stages)" % r["stages"] if r["sync"] == "pingpong"
                                else "k_gemm_win (split-window ring)" if r["stages"] == 5
                                else "k_gemm (%s, %d stages)" % (r["sync"], r["stages"]))},
    }
    if not args.no_reference:
        line["reference"] = reference_matmul(dA, dB, C, w, args.steps, args.warmup, torch)
    if not args.no_workloads:
        line["workloads"] = other_workloads(bd, w.name, args, torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
