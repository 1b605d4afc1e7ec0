#!/usr/bin/env python3
"""Throughput of the pipelined persistent bf16 GEMM on one MI355X.

A step is one C = A * B over the whole throughput workload (8192 x 8192 x 8192,
B stored N x K, seeded uniform[-1, 1) bf16 inputs already resident in HBM).
Every (sync scheme, ring stages) configuration of the library is timed on it
-- barrier sync at 2, 3 and 4 stages and over the split-window ring
(stages 5), flag sync at 2, 3 and 4, the wave-specialised and the ping-pong
kernels at 2, 3 and 4 -- and ``value`` is the fastest.  The other four
workloads get the same matrix under ``workloads``.  Prints one JSON line.

Also reports:
  roofline      achieved matrix-core TFLOP/s of the fastest configuration's
                GEMM kernel (2*M*N*K per call / mean time per call from HIP
                events on the launch stream before the first and after the
                last timed call) against the dense bf16 peak, plus
                HBM traffic per launch from the committed rocprofv3 counter
                summary when it matches the current kernel source;
  clock         per configuration, the mean shader clock of its kernels in
                the committed counter pass (GRBM_GUI_ACTIVE per XCD over the
                dispatch's duration), and the fraction of the peak at that
                clock (256 CU x 4096 FLOP/clk x clock);
  ceiling       what the matrix cores sustain under the board's power limit
                on the same kind of operand data with no memory traffic at
                all (gemm_probe_mfma_ceiling, at the GEMM kernels' wave shape,
                fragments in registers or re-read from LDS), beside the same
                loop on all-zero operands;
  sustained     the fastest configuration run back to back for several seconds
                (--sustain-seconds) in batches timed with HIP events: the
                throughput once the clock has settled for seconds, and the
                spread between batches;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same product
                (a few rows of C), on the host cores it actually uses; each
                other workload's oracle sample is under its entry;
  reference     torch.matmul (hipBLASLt) on the same operands in the same
                process, as context only.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sync all|barrier|flags|wavespec|pingpong]
                       [--stages S] [--workload NAME] [--no-cpu-baseline] [--no-workloads] ...
       python bench.py --counter-run            (a short pass over every configuration, for rocprofv3 --pmc)
       python bench.py --summarize-counters SQ_CSV FETCH_CSV WRITE_CSV MANIFEST_JSON [TCC_CSV]   (no GPU)
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
PEAK_CLOCK_GHZ = 2.4
FLOP_PER_CLK_GPU = 256 * 4096
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCE = os.path.join(ROOT, "pipelined_tiled_dense_amd", "csrc", "gemm_bf16.hip")
HEADLINE = "gemm8192_nk"
COPY_BYTES = 1 << 30

SYNC_NAMES = {0: "barrier", 1: "flags", 2: "wavespec", 3: "pingpong"}
# Every (sync mode, stages) configuration the library offers; stages 5 is the
# split-window ring.  They run in this order on every workload: the first
# launches of a process meet a cool chip whose clock then settles under the
# power limit, so the slowest kernels go first.
CONFIGS = [("pingpong", 2), ("pingpong", 3), ("pingpong", 4),
           ("wavespec", 2), ("wavespec", 3), ("wavespec", 4),
           ("flags", 2), ("flags", 3), ("flags", 4),
           ("barrier", 3), ("barrier", 4), ("barrier", 5), ("barrier", 2)]
DEFAULT_STAGES = {"barrier": 5, "flags": 2, "wavespec": 2, "pingpong": 3}


def label(sync, stages):
    return "%s/%d" % (sync, stages)


def timed_configs(workload):
    """The (sync, stages) runs bench.py times on a workload, in run order.
    The full-size parity tests check exactly these."""
    return list(CONFIGS)


def kernel_sha():
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sync", default="all", choices=["all", "barrier", "flags", "wavespec", "pingpong"])
    ap.add_argument("--stages", type=int, default=0, help="with --sync: one stage count (0: the mode's default)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the headline workload's oracle sample")
    ap.add_argument("--cpu-seconds-other", type=float, default=2.5,
                    help="target CPU time of each other workload's oracle sample")
    ap.add_argument("--no-reference", action="store_true", help="skip the torch.matmul timing")
    ap.add_argument("--sustain-seconds", type=float, default=8.0,
                    help="run the fastest configuration back to back for this long after the timed steps "
                         "and report it as `sustained` (0: skip)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the matrix-core ceiling probe")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other configurations")
    ap.add_argument("--counter-run", action="store_true",
                    help="a short, untimed pass over every workload and configuration (plus a 1 GiB "
                         "device copy for the counter calibration), writing the dispatch manifest")
    ap.add_argument("--manifest", default=None, help="where --counter-run writes its manifest")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_TRACE_CSV", "BENCH_JSON"),
                    help="turn a rocprofv3 kernel trace of a bench.py run into the committed summary (no GPU)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="turn the rocprofv3 counter CSVs of --counter-run passes into the committed "
                         "summary (no GPU needed)")
    return ap.parse_args(argv)


# -- counter summary (host only) --------------------------------------------------
def _dispatches(path):
    """rocprofv3 counter_collection CSV -> list of dispatches in order:
    (kernel name, duration ns, {counter: value summed over instances})."""
    import csv
    per = {}
    for row in csv.DictReader(open(path)):
        d = per.setdefault(int(row["Dispatch_Id"]), {
            "name": row["Kernel_Name"],
            "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"]),
            "c": {}})
        d["c"][row["Counter_Name"]] = d["c"].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return [per[k] for k in sorted(per)]


_FAMILY = None


def kernel_family(name):
    """Which of the library's kernels a demangled name is ('k_gemm_ws', ...),
    or None for kernels that are not the library's."""
    global _FAMILY
    if _FAMILY is None:
        import re
        _FAMILY = re.compile(r"(?:^|[^A-Za-z0-9_])(k_gemm_win|k_gemm_ws|k_gemm_pp|k_reduce_splits|k_gemm|"
                             r"k_mfma_ceiling)<")
    m = _FAMILY.search(name)
    return m.group(1) if m else None


def kernel_config(name):
    """("sync/stages", B stored N x K) of a GEMM kernel name, read from its
    Cfg<BM, BN, BK, S, WM, WN, SYNC, B_NxK, loader waves, windows, MFMA block>
    (the split-window ring reports stages 5), or None."""
    i = name.find("Cfg<")
    if i < 0 or kernel_family(name) not in ("k_gemm", "k_gemm_win", "k_gemm_ws", "k_gemm_pp"):
        return None
    f = [x.strip() for x in name[i + 4:name.index(">", i)].split(",")]
    stages = 5 if f[9] == "true" else int(f[3])
    return label(SYNC_NAMES[int(f[6])], stages), f[7] == "true"


def _assign(dispatches, manifest):
    """Walk the library's dispatches in order against the manifest of calls.
    Returns {(workload, label): [dispatch lists, one per call]} and the other
    kernels dispatched before the first GEMM (the copy calibration's)."""
    lib = [d for d in dispatches if kernel_family(d["name"])]
    first = next((i for i, d in enumerate(dispatches) if kernel_family(d["name"])), len(dispatches))
    other = dispatches[:first]
    out = {}
    i = 0
    for e in manifest["calls"]:
        key = (e["workload"], e["config"])
        for _ in range(e["calls"]):
            grp = lib[i:i + len(e["kernels"])]
            fams = [kernel_family(d["name"]) for d in grp]
            if fams != e["kernels"]:
                raise SystemExit("dispatch %d: expected %s for %s, found %s" % (i, e["kernels"], key, fams))
            out.setdefault(key, []).append(grp)
            i += len(grp)
    if i != len(lib):
        raise SystemExit("%d library dispatches left over after the manifest" % (len(lib) - i))
    return out, other


def summarize_counters(paths, out_path=COUNTERS_FILE):
    """paths: SQ_CSV FETCH_CSV WRITE_CSV MANIFEST [TCC_CSV] -- the CSVs of
    the counter passes over --counter-run, its manifest, and optionally the
    pass with the L2 request, hit and miss counts."""
    if len(paths) not in (4, 5):
        raise SystemExit("--summarize-counters SQ_CSV FETCH_CSV WRITE_CSV MANIFEST [TCC_CSV]")
    sq_csv, fetch_csv, write_csv, manifest_path = paths[:4]
    manifest = json.load(open(manifest_path))
    sq, _ = _assign(_dispatches(sq_csv), manifest)
    fe, fe_other = _assign(_dispatches(fetch_csv), manifest)
    wr, wr_other = _assign(_dispatches(write_csv), manifest)
    tcc = _assign(_dispatches(paths[4]), manifest)[0] if len(paths) == 5 else None
    # The 1 GiB device copy is the largest copy kernel ahead of the first GEMM
    # (the first workload's small host-to-device copies may follow it).
    copy_f = max((d["c"]["FETCH_SIZE"] for d in fe_other if "FETCH_SIZE" in d["c"] and "copy" in d["name"].lower()),
                 default=0.0)
    copy_w = max((d["c"]["WRITE_SIZE"] for d in wr_other if "WRITE_SIZE" in d["c"] and "copy" in d["name"].lower()),
                 default=0.0)
    if copy_f <= 0 or copy_w <= 0:
        raise SystemExit("no copy-kernel dispatches for the calibration")
    # FETCH_SIZE and WRITE_SIZE are in KiB; scale each by the ratio of the
    # bytes a 1 GiB device copy moves to what the counter reads for it.
    f_scale = COPY_BYTES / (copy_f * 1024.0)
    w_scale = COPY_BYTES / (copy_w * 1024.0)
    entries = {}
    for (wl, cfg), calls in sq.items():
        main = [c[0] for c in calls]                       # the GEMM kernel of each call
        n = len(main)
        mean = lambda f: sum(f(d) for d in main) / n
        dur_ns = mean(lambda d: d["ns"])
        grbm = mean(lambda d: d["c"].get("GRBM_GUI_ACTIVE", 0.0)) / 8.0      # per XCD
        clock = grbm / dur_ns if dur_ns else 0.0
        busy = mean(lambda d: d["c"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0))
        lds_act = mean(lambda d: d["c"].get("SQ_LDS_IDX_ACTIVE", 0.0))
        bank = mean(lambda d: d["c"].get("SQ_LDS_BANK_CONFLICT", 0.0))
        call_bytes = lambda groups, ctr, scale: sum(sum(d["c"].get(ctr, 0.0) for d in g) for g in groups) \
            / len(groups) * 1024.0 * scale
        fetch = call_bytes(fe[(wl, cfg)], "FETCH_SIZE", f_scale)
        write = call_bytes(wr[(wl, cfg)], "WRITE_SIZE", w_scale)
        entries.setdefault(wl, {})[cfg] = {
            "kernel": main[0]["name"],
            "kernels_per_call": [kernel_family(d["name"]) for d in calls[0]],
            "dispatches": n,
            "duration_us": round(dur_ns / 1e3, 2),
            "clock_ghz": round(clock, 4),
            "mfma_busy": round(busy / (grbm * 1024.0), 4) if grbm else None,
            "mfma_insts": mean(lambda d: d["c"].get("SQ_INSTS_MFMA", 0.0)),
            "lds_insts": mean(lambda d: d["c"].get("SQ_INSTS_LDS", 0.0)),
            "salu_insts": mean(lambda d: d["c"].get("SQ_INSTS_SALU", 0.0)),
            "vmem_rd_insts": mean(lambda d: d["c"].get("SQ_INSTS_VMEM_RD", 0.0)),
            "lds_bank_conflict_of_active": round(bank / lds_act, 5) if lds_act else None,
            "lds_active_of_cycles": round(lds_act / (grbm * 256.0), 4) if grbm else None,
            "fetch_bytes_per_call": round(fetch),
            "write_bytes_per_call": round(write),
            "hbm_bytes_per_call": round(fetch + write),
        }
        if tcc is not None:
            # The GEMM kernel's own L2 traffic (a split call's reduction is
            # not counted here), in 128-byte requests.
            gemm = [c[0] for c in tcc[(wl, cfg)]]
            req = sum(d["c"].get("TCC_REQ_sum", 0.0) for d in gemm) / len(gemm)
            miss = sum(d["c"].get("TCC_MISS_sum", 0.0) for d in gemm) / len(gemm)
            entries[wl][cfg].update({"l2_requests": req, "l2_misses": miss,
                                     "l2_miss_rate": round(miss / req, 4) if req else None})
    out = {"kernel_source_sha256": kernel_sha(),
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_scale": f_scale, "write_scale": w_scale,
                           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w},
           "entries": entries}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    if out_path == COUNTERS_FILE:
        write_counter_reports(out)
    print(json.dumps({"written": out_path, "workloads": sorted(entries)}))
    return out


PROFILES = os.path.join(ROOT, "profiles")
COUNTER_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp   # then, from the repository root:",
    "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM_RD "
    "SQ_INSTS_VALU SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE --output-format csv -d <out>/sq -o sq "
    "-- python3 bench.py --counter-run --manifest <out>/manifest.json",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o fetch -- python3 bench.py --counter-run "
    "--manifest <out>/manifest.json",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o write -- python3 bench.py --counter-run "
    "--manifest <out>/manifest.json",
    "rocprofv3 --pmc TCC_REQ_sum TCC_HIT_sum TCC_MISS_sum --output-format csv -d <out>/tcc -o tcc -- python3 "
    "bench.py --counter-run --manifest <out>/manifest.json",
    "python3 bench.py --summarize-counters <out>/sq/sq_counter_collection.csv "
    "<out>/fetch/fetch_counter_collection.csv <out>/write/write_counter_collection.csv <out>/manifest.json "
    "<out>/tcc/tcc_counter_collection.csv",
]


def write_counter_reports(info, out_dir=PROFILES):
    """One markdown table per workload from the counter summary, with the
    kernels' names exactly as rocprofv3 reports them."""
    from pipelined_tiled_dense_amd.inputs import WORKLOADS
    cal = info["calibration"]
    paths = []
    for wl, cfgs in info["entries"].items():
        w = WORKLOADS.get(wl)
        title = ("%s (%d x %d x %d, B stored %s)" % (wl, w.M, w.N, w.K, "N x K" if w.b_transposed else "K x N")
                 if w else "matrix-core ceiling probe (gemm_probe_mfma_ceiling, 256 workgroups, 1024 iterations)")
        lines = ["# Counters: %s, every sync mode and stage count" % title, "",
                 "Kernel source sha256 `%s`.  Commands (one counter group per pass; each pass runs the same "
                 "short, untimed sequence of calls, 4 per configuration, and the summary attributes every "
                 "dispatch through the manifest that sequence writes):" % info["kernel_source_sha256"], "", "```"]
        lines += COUNTER_COMMANDS + ["```", "",
                 "Per call, mean over the 4 calls: duration of the GEMM kernel (or the probe); clock = "
                 "GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x "
                 "1024 SIMDs); bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; instruction counts are "
                 "per call, whole GPU; HBM bytes = FETCH_SIZE x %.4f + WRITE_SIZE x %.4f (KiB), the factors that "
                 "make a 1 GiB device copy read and write 1 GiB, summed over every kernel of the call (a split "
                 "call's reduction included).  L2 requests (128 bytes each) and the fraction that missed are "
                 "TCC_REQ_sum and TCC_MISS_sum of the GEMM kernel alone.  Calls shorter than a few microseconds "
                 "give meaningless clocks."
                 % (cal["fetch_scale"], cal["write_scale"]), "",
                 "| config | kernel (as rocprofv3 names it) | duration (us) | clock (GHz) | MFMA busy | SALU instr | "
                 "LDS instr | VMEM read instr | LDS bank conflicts | HBM read (GB) | HBM write (GB) | L2 requests | "
                 "L2 miss rate |",
                 "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        fmt = lambda v, f: "-" if v is None else f % v
        for cfg, e in cfgs.items():
            lines.append("| %s | `%s` | %.1f | %.3f | %s | %.3g | %.3g | %.3g | %s | %.3f | %.3f | %s | %s |" % (
                cfg, e["kernel"], e["duration_us"], e["clock_ghz"], fmt(e["mfma_busy"], "%.3f"), e["salu_insts"],
                e["lds_insts"], e["vmem_rd_insts"], fmt(e["lds_bank_conflict_of_active"], "%.4f"),
                e["fetch_bytes_per_call"] / 1e9, e["write_bytes_per_call"] / 1e9,
                fmt(e.get("l2_requests"), "%.3g"), fmt(e.get("l2_miss_rate"), "%.3f")))
        path = os.path.join(out_dir, "%s_counters.md" % wl)
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        paths.append(path)
    return paths


def summarize_trace(trace_csv, bench_json, out_path=None, workload=HEADLINE):
    """Kernel-trace summary of a bench.py run: per configuration of the
    headline workload, the GEMM kernel's dispatches (warm-up included) and
    their mean duration, beside the mean per-call time the same run measured
    with HIP events.  The headline workload is the only one with B stored
    N x K, so its kernels are told apart by name."""
    import csv
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    per = {}
    order = []
    for row in csv.DictReader(open(trace_csv)):
        name = row["Kernel_Name"]
        ns = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
        if name not in per:
            per[name] = []
            order.append(name)
        per[name].append(ns)
    out_path = out_path or os.path.join(PROFILES, "%s_kernel_trace.md" % workload)
    lines = ["# Kernel trace: %s, every sync mode and stage count" % workload, "",
             "Command (from the repository root, with TMPDIR=/tmp):", "", "```",
             "rocprofv3 --kernel-trace --stats --output-format csv -d <out>/kt -o kt -- python3 bench.py "
             "--steps %d --warmup %d --no-cpu-baseline > <out>/kt_bench.json" % (line["steps"], line["warmup"]),
             "python3 bench.py --summarize-trace <out>/kt/kt_kernel_trace.csv <out>/kt_bench.json", "```", "",
             "Kernel source sha256 `%s`.  Per configuration: the dispatches of its kernel in the trace "
             "(%d warm-up, %d timed and %d clock-sampled calls), their mean and minimum duration, the mean "
             "per-call time bench.py measured in the same run (HIP events on the launch stream before the first "
             "and after the last timed call; the roofline's `achieved` uses it), and the clock sampled inside the kernels in the calls right "
             "after the timed ones, with the MFMA-busy fraction it implies (TFLOP/s over 1,048,576 FLOP per "
             "clock)." % (kernel_sha(), line["warmup"], line["steps"], CLOCK_SAMPLE_CALLS), "",
             "| config | kernel (as rocprofv3 names it) | dispatches | trace mean (us) | trace min (us) | "
             "HIP events mean (us) | TFLOP/s (events) | clock (GHz) | MFMA busy |",
             "|---|---|---|---|---|---|---|---|---|"]
    for cfg, e in line["modes"].items():
        cands = [n for n in order if kernel_config(n) == (cfg, True)]
        for n in cands:
            d = per[n]
            lines.append("| %s | `%s` | %d | %.1f | %.1f | %.1f | %.1f | %s | %s |" % (
                cfg, n, len(d), sum(d) / len(d) / 1e3, min(d) / 1e3, e["kernel_ms_mean"] * 1e3, e["tflops"],
                e.get("clock_ghz", "-"), e.get("mfma_busy", "-")))
    lines += ["", "The run's line: value %.2f TFLOP/s (%s), roofline achieved %.2f TFLOP/s, frac %.4f."
              % (line["value"], line["roofline"]["kernel"], line["roofline"]["achieved"], line["roofline"]["frac"])]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


def counters_for(workload, cfg, path=COUNTERS_FILE):
    """The committed counter entry of a workload's configuration, or None when
    there is none or it was taken on another kernel source."""
    try:
        info = json.load(open(path))
    except (OSError, ValueError):
        return None
    if info.get("kernel_source_sha256") != kernel_sha():
        return None
    return info.get("entries", {}).get(workload, {}).get(cfg)


# -- GPU legs ---------------------------------------------------------------------
def time_mode(bd, dA, dB, C, w, sync, stages, steps, warmup, torch):
    """`warmup` untimed calls, then exactly `steps` calls timed between two
    synchronisations: the wall clock around them, and HIP events recorded on
    the launch stream before the first and after the last.  No events go
    between the calls: each would put a marker between two kernels, which
    measured 2-4 us per call on the GPU.  Returns (wall seconds, mean ms per
    call on the GPU)."""
    for _ in range(warmup):
        bd.gemm(dA, dB, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        bd.gemm(dA, dB, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / steps


CLOCK_SAMPLE_CALLS = 10


def sampled_clock(bd, dA, dB, C, w, sync, stages, calls=CLOCK_SAMPLE_CALLS):
    """The clock the GEMM kernels ran at over `calls` further calls, from the
    library's in-kernel samples (elapsed s_memtime over elapsed s_memrealtime
    per workgroup), in GHz; None without samples.  Run right after a timed
    loop, so the board is in the same power state."""
    bd.gemm_bf16_clock_samples(reset=True)
    prev = bd.gemm_bf16_set_clock_sampling(True)
    try:
        for _ in range(calls):
            bd.gemm(dA, dB, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
        got = bd.gemm_bf16_clock_samples(reset=True)
    finally:
        bd.gemm_bf16_set_clock_sampling(prev)
    return got["clock_ghz"]


def measure_workload(bd, w, configs, args, torch, A=None, B=None):
    """Every configuration on one workload: mean time per call from HIP events
    on the launch stream around the timed calls, wall-clock throughput, % of peak,
    the clock sampled inside the kernels right after the timed loop and the
    MFMA-busy fraction it implies (FLOP rate over 1,048,576 FLOP per clock;
    for split calls the reduction kernel's time counts as not busy), and, where
    the committed counter summary has them, the counter pass's clock and the
    call's HBM traffic with the rate it gives at this run's time."""
    from pipelined_tiled_dense_amd.inputs import workload_operands
    if A is None:
        A, B = workload_operands(w)
    dA, dB = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * w.M * w.N * w.K
    res = {}
    for sync, stages in configs:
        plan = bd.gemm_bf16_plan(w.M, w.N, w.K, w.b_transposed, stages, bd.SYNC_MODES[sync])
        wall, mean_ms = time_mode(bd, dA, dB, C, w, sync, stages, args.steps, args.warmup, torch)
        tf = flops / (mean_ms * 1e-3) / 1e12
        e = {"tflops": round(tf, 2), "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
             "wall_tflops": round(flops / (wall / args.steps) / 1e12, 2),
             "ms_per_step": round(wall * 1e3 / args.steps, 4),
             "kernel_ms_mean": round(mean_ms, 4),
             "tile": "%dx%dx%d" % (plan["bm"], plan["bn"], plan["bk"]), "grid": plan["grid"],
             "k_splits": plan["k_splits"], "tail_tiles": plan["tail_tiles"], "mfma_block": plan["mfma_block"]}
        ghz = sampled_clock(bd, dA, dB, C, w, sync, stages)
        if ghz:
            e["clock_ghz"] = round(ghz, 3)
            e["mfma_busy"] = round(tf * 1e12 / (FLOP_PER_CLK_GPU * ghz * 1e9), 4)
        cnt = counters_for(w.name, label(sync, stages))
        if cnt and cnt.get("clock_ghz"):
            e["counter_clock_ghz"] = cnt["clock_ghz"]
            e["frac_of_peak_at_counter_clock"] = round(tf * 1e12 / (FLOP_PER_CLK_GPU * cnt["clock_ghz"] * 1e9), 4)
            e["counter_mfma_busy"] = cnt.get("mfma_busy")
        if cnt and cnt.get("hbm_bytes_per_call"):
            # HBM bytes of the counter pass per call, and the rate they give at
            # this run's per-call time
            e["hbm_gb_per_call"] = round(cnt["hbm_bytes_per_call"] / 1e9, 4)
            e["hbm_gbps"] = round(cnt["hbm_bytes_per_call"] / (mean_ms * 1e-3) / 1e9, 1)
        res[label(sync, stages)] = e
        print("# %s %s: %s" % (w.name, label(sync, stages), json.dumps(e)), file=sys.stderr, flush=True)
    return res, (A, B, dA, dB, C)


# Untimed calls before torch.matmul is timed: measured at 8192^3, hipBLASLt's
# kernel needs about 50 calls after another kernel ran before its throughput
# settles (its first 25 ran ~13% below its steady state), against about 20
# for ours, which run after the other configurations anyway.
REFERENCE_WARMUP = 100


def sustained(bd, w, sync, stages, dA, dB, C, seconds, torch, batch=100):
    """The fastest configuration run back to back for about `seconds`, in
    batches of `batch` calls, each batch between one pair of HIP events on the
    launch stream: the throughput once the board's clock has settled under its
    power limit for seconds rather than milliseconds, and how much it moves
    from batch to batch.  Also keeps the GPU visibly busy for that long."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rates, total_ms, calls = [], 0.0, 0
    while total_ms < 1000.0 * seconds:
        e0.record()
        for _ in range(batch):
            bd.gemm(dA, dB, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        total_ms += ms
        calls += batch
        rates.append(2.0 * w.M * w.N * w.K * batch / ms / 1e9)
    return {"config": label(sync, stages), "seconds": round(total_ms / 1e3, 2), "calls": calls,
            "tflops": round(2.0 * w.M * w.N * w.K * calls / total_ms / 1e9, 2),
            "batch_tflops_min": round(min(rates), 2), "batch_tflops_max": round(max(rates), 2),
            "pct_of_peak": round(100.0 * 2.0 * w.M * w.N * w.K * calls / total_ms / 1e9 / PEAK_BF16_TFLOPS, 2)}


def reference_matmul(dA, dB, C, w, steps, warmup, torch):
    """torch.matmul on the same operands (B^T as a view when B is stored N x K),
    after max(warmup, REFERENCE_WARMUP) untimed calls."""
    Bop = dB.t() if w.b_transposed else dB
    for _ in range(max(warmup, REFERENCE_WARMUP)):
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


# Variants of the matrix-core ceiling probe: name -> (waves, fragments from
# LDS, all-zero data).  8 waves of 128 x 64 is the all-wave kernels' layout,
# 4 waves of 128 x 128 the layout with a third fewer LDS reads per MFMA, and
# 4 waves of 128 x 64 (waves = -4) the wave-specialised kernel's MFMA waves,
# one per SIMD.
CEILING_VARIANTS = {"w8_registers_zero_data": (8, 0, True), "w8_registers": (8, 0, False),
                    "w8_lds_reads": (8, 1, False), "w4_registers": (4, 0, False), "w4_lds_reads": (4, 1, False),
                    "w4x64_registers": (-4, 0, False), "w4x64_lds_reads": (-4, 1, False)}


def ceiling_flop_per_block_iter(variant):
    waves = CEILING_VARIANTS[variant][0]
    return 1 << (22 if waves == -4 else 23)
CEILING_ITERS = 1024
CEILING_BLOCKS = 256
# Untimed calls before each variant (about 1 ms each): the clock settles tens
# of milliseconds after the load changes, and the variants draw different power.
CEILING_WARMUP = 30


def _ceiling_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "pipelined_tiled_dense_amd", "libgemm_probes.so"))
    lib.gemm_probe_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]
    lib.gemm_probe_mfma_ceiling.restype = ctypes.c_int
    return lib


def _ceiling_call(torch, lib, variant, data, sink, stamps=None):
    waves, from_lds, _ = CEILING_VARIANTS[variant]
    rc = lib.gemm_probe_mfma_ceiling(data.data_ptr(), data.numel(), from_lds, waves, CEILING_ITERS, CEILING_BLOCKS,
                                     sink.data_ptr(), stamps.data_ptr() if stamps is not None else None,
                                     torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError("gemm_probe_mfma_ceiling failed: %d" % rc)


def _ceiling_data(torch):
    g = torch.Generator(device="cpu").manual_seed(12345)
    rand = (torch.rand(1 << 22, generator=g) * 2 - 1).to(torch.bfloat16).cuda()
    zero = torch.zeros(1 << 22, dtype=torch.bfloat16, device="cuda")
    sink = torch.empty(CEILING_BLOCKS * 512, dtype=torch.float32, device="cuda")
    return rand, zero, sink


def mfma_ceiling(torch, steps=20):
    """gemm_probe_mfma_ceiling on 256 workgroups in every variant: TFLOP/s
    from HIP events (2^23 FLOP per workgroup-iteration), with the counter
    pass's clock and MFMA busy where the committed summary has them."""
    lib = _ceiling_lib()
    rand, zero, sink = _ceiling_data(torch)
    stream = torch.cuda.current_stream()
    stamps = torch.zeros((steps, CEILING_BLOCKS, 2), dtype=torch.int64, device="cuda")
    rt_hz = wall_clock_hz(torch)
    out = {}
    for name, (_, _, zero_data) in CEILING_VARIANTS.items():
        data = zero if zero_data else rand
        for _ in range(CEILING_WARMUP):
            _ceiling_call(torch, lib, name, data, sink)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
        for i in range(steps):
            ev[2 * i].record(stream)
            _ceiling_call(torch, lib, name, data, sink, stamps[i])
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / steps
        flop = float(CEILING_BLOCKS) * ceiling_flop_per_block_iter(name) * CEILING_ITERS
        tf = flop / (ms * 1e-3) / 1e12
        st = stamps.double().sum(dim=(0, 1))
        clock = float(st[0] / st[1]) * rt_hz / 1e9 if float(st[1]) > 0 else None
        e = {"tflops": round(tf, 1), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "ms": round(ms, 4),
             "clock_ghz_memtime": round(clock, 3) if clock else None,
             "mfma_busy_at_that_clock": round(tf * 1e12 / (FLOP_PER_CLK_GPU * clock * 1e9), 3) if clock else None}
        cnt = counters_for("ceiling", name)
        if cnt and cnt.get("clock_ghz"):
            e["counter_clock_ghz"] = cnt["clock_ghz"]
            e["counter_mfma_busy"] = cnt.get("mfma_busy")
        out[name] = e
    out["note"] = ("MFMA-only loop of 16x16x32 bf16 at the GEMM kernels' wave shapes, 256 workgroups, no global "
                   "memory traffic; random uniform[-1,1) bf16 operands unless named zero_data")
    out["lds_read_bandwidth"] = lds_read_bandwidth(torch)
    return out


LDS_BW_ITERS = 4096


def lds_read_bandwidth(torch):
    """gemm_probe_lds_read_bw on 256 workgroups (one per compute unit): the
    LDS read bandwidth of a CU in bytes per shader clock, from each
    workgroup's own s_memtime stamps around its reads.  The swizzles and the
    LDS budget of the kernels assume 64 four-byte banks, 256 bytes per clock."""
    import ctypes
    lib = _ceiling_lib()
    lib.gemm_probe_lds_read_bw.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p]
    lib.gemm_probe_lds_read_bw.restype = ctypes.c_int
    blocks = 256
    sink = torch.empty(blocks * 1024, dtype=torch.int32, device="cuda")
    stamps = torch.zeros((blocks, 2), dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        if lib.gemm_probe_lds_read_bw(LDS_BW_ITERS, blocks, sink.data_ptr(), stamps.data_ptr(), s) != 0:
            raise RuntimeError("gemm_probe_lds_read_bw failed")
    torch.cuda.synchronize()
    ticks = stamps[:, 0].double().cpu()
    bpc = (LDS_BW_ITERS + 1) * 128 * 1024 / ticks
    return {"bytes_per_clk_per_cu": round(float(bpc.mean()), 1), "min": round(float(bpc.min()), 1),
            "max": round(float(bpc.max()), 1), "of_256": round(float(bpc.mean()) / 256.0, 4)}


def wall_clock_hz(torch):
    """Tick rate of s_memrealtime (the device's constant-rate wall clock)."""
    import ctypes
    lib = _ceiling_lib()
    lib.gemm_probe_wall_clock_hz.argtypes = []
    lib.gemm_probe_wall_clock_hz.restype = ctypes.c_int64
    hz = lib.gemm_probe_wall_clock_hz()
    return float(hz) if hz > 0 else 100e6


def cpu_baseline(w, A, B, target_s):
    import numpy as np

    import oracle
    from pipelined_tiled_dense_amd.inputs import bits
    o = oracle.load()
    Ab, Bb = bits(A), bits(B)
    threads = o.num_threads()
    # calibrate on a few rows, then run a sample sized for ~target_s seconds
    cal_rows = max(1, min(w.M, threads))
    t0 = time.perf_counter()
    o.gemm_bf16(np.ascontiguousarray(Ab[:cal_rows]), Bb, w.b_transposed)
    t_cal = time.perf_counter() - t0
    rows = int(max(cal_rows, min(w.M, cal_rows * target_s / max(t_cal, 1e-6))))
    rows = min(w.M, max(cal_rows, (rows // threads) * threads))
    t0 = time.perf_counter()
    o.gemm_bf16(np.ascontiguousarray(Ab[:rows]), Bb, w.b_transposed)
    t = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / t / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "rows 0..%d of C (%d x %d x %d, %.3g GFLOP) in %.2f s; fp64 triple loop, "
                      "one bf16 rounding" % (rows - 1, rows, w.N, w.K, flops / 1e9, t),
            "host": host_cpu()}


def host_cpu():
    """The host CPU the oracle ran on: model name and the cores this process
    may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count()
    return {"model": model, "cores_allowed": allowed}


def counter_run(bd, args, torch):
    """Every configuration on every workload, 1 warm-up call and 3 counted
    calls each, after a 1 GiB device copy: the command the rocprofv3 --pmc
    passes profile.  The manifest lists the calls in order with the library
    kernels each launches, so the summary can attribute every dispatch."""
    from pipelined_tiled_dense_amd.inputs import WORKLOADS, workload_operands
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    calls = []
    for name, w in WORKLOADS.items():
        A, B = workload_operands(w)
        dA, dB = A.cuda(), B.cuda()
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        for sync, stages in timed_configs(name):
            pl = bd.gemm_bf16_plan(w.M, w.N, w.K, w.b_transposed, stages, bd.SYNC_MODES[sync])
            fam = {"barrier": "k_gemm_win" if stages == 5 else "k_gemm", "flags": "k_gemm",
                   "wavespec": "k_gemm_ws", "pingpong": "k_gemm_pp"}[sync]
            kernels = [fam] + ([fam] if pl["tail_tiles"] > 0 else []) + \
                      (["k_reduce_splits"] if pl["k_splits"] > 1 or pl["tail_tiles"] > 0 else [])
            for _ in range(4):
                bd.gemm(dA, dB, b_transposed=w.b_transposed, sync=sync, stages=stages, out=C)
            torch.cuda.synchronize()
            calls.append({"workload": name, "config": label(sync, stages), "calls": 4, "kernels": kernels})
        del dA, dB, C
    lib = _ceiling_lib()
    rand, zero, sink = _ceiling_data(torch)
    for name, (_, _, zero_data) in CEILING_VARIANTS.items():
        for _ in range(4):
            _ceiling_call(torch, lib, name, zero if zero_data else rand, sink)
        torch.cuda.synchronize()
        calls.append({"workload": "ceiling", "config": name, "calls": 4, "kernels": ["k_mfma_ceiling"]})
    path = args.manifest or os.path.join(ROOT, "counter_out", "counter_manifest.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"calls": calls}, f, indent=1)
    print(json.dumps({"manifest": path, "calls": len(calls)}), flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GEMM has no multi-GPU path in this build "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from pipelined_tiled_dense_amd import binding as bd
    from pipelined_tiled_dense_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    bd.library()
    if args.counter_run:
        counter_run(bd, args, torch)
        return

    w = WORKLOADS[args.workload]
    if args.sync == "all":
        configs = timed_configs(w.name)
    else:
        configs = [(args.sync, args.stages or DEFAULT_STAGES[args.sync])]
    results, (A, B, dA, dB, C) = measure_workload(bd, w, configs, args, torch)
    timeouts = bd.gemm_bf16_sync_timeouts()
    best = max(results, key=lambda k: results[k]["wall_tflops"])
    r = results[best]
    sync, stages = best.split("/")[0], int(best.split("/")[1])
    achieved = r["tflops"]
    cnt = counters_for(w.name, best)
    kernel = {"wavespec": "k_gemm_ws", "pingpong": "k_gemm_pp"}.get(sync, "k_gemm_win" if stages == 5 else "k_gemm")
    line = {
        "metric": "bf16 GEMM TFLOP/s and % of MFMA peak at 1 GPU (8192^3, per sync mode)",
        "value": r["wall_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "b_layout": "N x K (K contiguous)" if w.b_transposed else "K x N",
                   "inputs": "seeded uniform[-1,1) rounded to bf16, seed %d" % w.seed,
                   "sync_mode": sync, "stages": stages, "tile": r["tile"], "grid": r["grid"],
                   "accumulate": "fp32", "output": "bf16 (RNE)"},
        "pct_of_peak": round(100.0 * r["wall_tflops"] / PEAK_BF16_TFLOPS, 2),
        "modes": results,
        "sync_timeouts": timeouts,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": cnt["hbm_bytes_per_call"] if cnt else None,
                     "kernel": "%s (%s)" % (kernel, best),
                     "clock_ghz_in_kernel": r.get("clock_ghz"), "mfma_busy_in_kernel": r.get("mfma_busy"),
                     "clock_ghz_counter_pass": cnt["clock_ghz"] if cnt else None,
                     "frac_at_counter_clock": r.get("frac_of_peak_at_counter_clock")},
    }
    if args.sustain_seconds > 0:
        line["sustained"] = sustained(bd, w, sync, stages, dA, dB, C, args.sustain_seconds, torch)
        print("# sustained: %s" % json.dumps(line["sustained"]), file=sys.stderr, flush=True)
    if not args.no_reference:
        line["reference"] = reference_matmul(dA, dB, C, w, args.steps, args.warmup, torch)
    del dA, dB, C
    if not args.no_ceiling:
        line["ceiling"] = mfma_ceiling(torch)
        print("# ceiling: %s" % json.dumps(line["ceiling"]), file=sys.stderr, flush=True)
    others = {}
    if not args.no_workloads:
        for name, ow in WORKLOADS.items():
            if name == w.name:
                continue
            res, (oA, oB, odA, odB, oC) = measure_workload(bd, ow, timed_configs(name), args, torch)
            b = max(res, key=lambda k: res[k]["tflops"])
            entry = {"M": ow.M, "N": ow.N, "K": ow.K, "b_layout": "N x K" if ow.b_transposed else "K x N",
                     "best": b, "tflops": res[b]["tflops"], "pct_of_peak": res[b]["pct_of_peak"],
                     "configs": res}
            if not args.no_reference:
                entry["reference_tflops"] = reference_matmul(odA, odB, oC, ow, args.steps, args.warmup,
                                                             torch)["tflops"]
            del odA, odB, oC
            others[name] = (entry, oA, oB)
        line["workloads"] = {k: v[0] for k, v in others.items()}
        line["sync_timeouts"] = bd.gemm_bf16_sync_timeouts()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_seconds)
        for name, (entry, oA, oB) in others.items():
            entry["cpu_baseline"] = cpu_baseline(WORKLOADS[name], oA, oB, args.cpu_seconds_other)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
