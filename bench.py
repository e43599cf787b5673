"""Benchmark of the row-major GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

One step is one SGEMM of 4096x4096x1024 (fp32) followed by one HGEMM of
4096x4096x4096 (fp16 inputs, fp32 accumulation and output), alpha = 1 and
beta = 0, on seeded uniform[-1,1) inputs already resident in HBM.  The value is
the step's throughput, (2*4096*4096*1024 + 2*4096^3) / step time, in TFLOPS;
the per-kernel TFLOPS and fraction of the MI355X peak for its dtype are
reported beside it, with the roofline of the dominant (longest) kernel taken
from HIP events recorded on the stream the kernels run on.  The CPU oracle is
timed on a bounded sample of the same workload as a baseline.  The other
benchmark configurations (SGEMM 512^3, the 1001x777x513 and 1024x1024x512
SGEMMs, HGEMM 2048^3 and 16 batched 1024^3 HGEMMs with beta = 1), two ragged
shapes and the transposed storage combinations are timed after the main run
and reported under "extra" (not part of the value).

Warm-up: under this load the clocks take about 40 ms (about 100 steps) to
settle; the default 200 untimed steps cover that, and 50 steps are timed.

Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS (2MNK/t) + % of dtype peak: SGEMM 4096x4096x1024, HGEMM 4096^3"
# MI355X peaks: 256 CUs x 2.4 GHz; fp32 matrix/vector 256 flop/clk/CU, fp16 dense MFMA 4096 flop/clk/CU.
PEAK_F32_TFLOPS = 157.3
PEAK_F16_TFLOPS = 2516.6
PEAK_BF16_TFLOPS = 2516.6   # bf16 dense MFMA runs at the fp16 rate
PEAK_HBM_GBS = 8000.0
_CSRC = "dense_gemm_optimisation_f32_amd/csrc/"
# the files whose code makes up each kernel (its source and the headers it includes)
KERNEL_SOURCES = {
    "sgemm": [_CSRC + f for f in ("sgemm_mfma.hip", "epilogue.h", "tile_order.h", "gemm_internal.h")],
    "hgemm": [_CSRC + f for f in ("hgemm_mfma.hip", "epilogue.h", "tile_order.h", "gemm_internal.h")],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
COPY_BYTES = 256 << 20   # size of the calibration copy (read and written)


def source_digest(kind: str) -> str:
    """Digest of a kernel's code: its files with comments and whitespace removed,
    so that a counter record stays valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic_records():
    """The JSON block of the committed counter summary (profiles/hbm_traffic.md)."""
    text = open(TRAFFIC_FILE).read()
    start = text.index("```json") + len("```json")
    return json.loads(text[start:text.index("```", start)])


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when it is missing or was taken on a different version of the kernel source."""
    try:
        rec = _traffic_records()[kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_digest(kind) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the chip's clocks settle only after some tens of milliseconds of this load
    # (about 100 steps); the warm-up covers that so the timed steps are steady
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other configurations")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle time budget")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy three times (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-calibration run into profiles/hbm_traffic.md; uses no GPU")
    ap.add_argument("--write-trace", nargs=3, metavar=("STATS_CSV", "TRACE_CSV", "BENCH_LOG"),
                    help="turn a rocprofv3 --kernel-trace --stats run of this script into "
                         "profiles/kernel_trace_sgemm4096x4096x1024_hgemm4096cube.md; uses no GPU")
    ap.add_argument("--write-counters", nargs="+", metavar="CSV",
                    help="turn rocprofv3 counter_collection.csv files of the step's kernels into "
                         "profiles/counters_sgemm4096x4096x1024_hgemm4096cube.md; uses no GPU")
    args = ap.parse_args()
    if args.write_traffic:
        return write_traffic(*args.write_traffic)
    if args.write_counters:
        return write_counters(args.write_counters)
    if args.write_trace:
        return write_trace(*args.write_trace)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_gemm_optimisation_f32_amd as dg
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dg.load_library()    # raises if the HIP library is not built: there is no fallback
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def upload(buf):
        return torch.from_numpy(np.ascontiguousarray(buf)).to(dev)

    # ---- inputs (resident in HBM before timing)
    Ms, Ns, Ks = 4096, 4096, 1024
    ps = si.gemm_problem(Ms, Ns, Ks, seed=42, with_c=False)
    sA, sB = upload(ps["A"]), upload(ps["B"])
    sC = torch.empty(Ms * Ns, dtype=torch.float32, device=dev)
    Mh = Nh = Kh = 4096
    ph = si.gemm_problem(Mh, Nh, Kh, in_dtype=np.float16, seed=42, with_c=False)
    hA, hB = upload(ph["A"]), upload(ph["B"])
    hC = torch.empty(Mh * Nh, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration:
        # uninitialised buffers: no fill kernel joins the counted dispatches
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # plain elementwise copy: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst

    def sgemm():
        dg.gemm_f32(Ms, Ns, Ks, 1.0, sA, Ks, sB, Ns, 0.0, sC, Ns, stream)

    def hgemm():
        dg.gemm_f16_f32acc(Mh, Nh, Kh, 1.0, hA, Kh, hB, Nh, 0.0, hC, Nh, stream)

    for _ in range(args.warmup):
        sgemm()
        hgemm()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        sgemm()
        ev[i][1].record(stream)
        hgemm()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_s = [e[0].elapsed_time(e[1]) * 1e-3 for e in ev]
    t_h = [e[1].elapsed_time(e[2]) * 1e-3 for e in ev]
    flop_s = 2.0 * Ms * Ns * Ks
    flop_h = 2.0 * Mh * Nh * Kh
    step_s = wall / args.steps
    value = (flop_s + flop_h) / step_s / 1e12

    def kernel_record(name, ts, flop, peak, workload, bytes_alg):
        avg = statistics.fmean(ts)
        return {
            "workload": workload,
            "avg_ms": avg * 1e3, "median_ms": statistics.median(ts) * 1e3, "min_ms": min(ts) * 1e3,
            "tflops": flop / avg / 1e12, "peak_tflops": peak, "frac_of_peak": flop / avg / 1e12 / peak,
            "algorithmic_flop": flop, "algorithmic_bytes": bytes_alg,
        }

    w_s = "SGEMM fp32 row-major 4096x4096x1024 alpha=1 beta=0"
    w_h = "HGEMM fp16->fp32 row-major 4096x4096x4096 alpha=1 beta=0"
    bytes_s = 4 * (Ms * Ks + Ks * Ns + Ms * Ns)
    bytes_h = 2 * (Mh * Kh + Kh * Nh) + 4 * Mh * Nh
    per_kernel = {
        "sgemm": kernel_record("sgemm", t_s, flop_s, PEAK_F32_TFLOPS, w_s, bytes_s),
        "hgemm": kernel_record("hgemm", t_h, flop_h, PEAK_F16_TFLOPS, w_h, bytes_h),
    }
    dom = max(per_kernel, key=lambda k: per_kernel[k]["avg_ms"])
    dk = per_kernel[dom]
    roofline = {
        "kernel": dom, "bound": "mfma", "achieved": dk["tflops"], "peak": dk["peak_tflops"],
        "unit": "TFLOP/s", "frac": dk["frac_of_peak"], "traffic": measured_traffic(dom, dk["workload"]),
        "algorithmic_flop_per_launch": dk["algorithmic_flop"],
    }
    other = "hgemm" if dom == "sgemm" else "sgemm"
    ok = per_kernel[other]
    roofline_other = {
        "kernel": other, "bound": "mfma", "achieved": ok["tflops"], "peak": ok["peak_tflops"],
        "unit": "TFLOP/s", "frac": ok["frac_of_peak"], "traffic": measured_traffic(other, ok["workload"]),
    }

    extra = {} if args.no_extra else run_extra(dg, si, np, torch, dev, stream)

    cpu = None if args.no_cpu else cpu_baseline(si, np, ps, ph, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32+f16(f32acc)", "data": "synthetic",
        "config": {"workload": "one SGEMM 4096x4096x1024 (fp32) + one HGEMM 4096^3 (fp16 in, fp32 "
                               "accumulate/out) per step, row-major, alpha=1 beta=0, seeded uniform[-1,1)",
                   "parallelism": "single GPU"},
        "per_kernel": per_kernel,
        "roofline": roofline,
        "roofline_other": roofline_other,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


TRACE_STEPS, TRACE_WARMUP = 50, 200


def write_trace(stats_csv: str, trace_csv: str, bench_log: str) -> int:
    """Kernel-trace summary of a profiled run of this script: rocprofv3's statistics over
    all launches, the same over the timed launches only (the last TRACE_STEPS of each
    kernel), and the bench line's own HIP-event averages for comparison."""
    import csv

    def short(n):
        return n.replace("mi355gemm::(anonymous namespace)::", "").split("(")[0]

    stats = list(csv.DictReader(open(stats_csv)))
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    line = next(l for l in open(bench_log) if l.startswith('{"metric"'))
    bench_line = json.loads(line)
    cmd = (f"cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof -o run -- "
           f"python3 $R/bench.py --no-cpu --no-extra --steps {TRACE_STEPS} --warmup {TRACE_WARMUP} "
           f"> $OUT/prof.log\n"
           f"python3 $R/bench.py --write-trace $OUT/prof/run_kernel_stats.csv "
           f"$OUT/prof/run_kernel_trace.csv $OUT/prof.log   # R = repository root, OUT = an output directory")
    out = ["# rocprofv3 kernel trace: bench step (SGEMM 4096x4096x1024 fp32 + HGEMM 4096^3 fp16->fp32)", "",
           "Commands (run on one MI355X):", "", "```", cmd, "```", "",
           "All launches (warm-up included):", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    out += ["", f"Timed launches only (the last {TRACE_STEPS} of each kernel), beside the bench line's "
                "HIP-event averages over the same steps:", "",
            "| kernel | launches | rocprofv3 average (us) | bench average (us) |", "|---|---|---|---|"]
    for name, v in per.items():
        kind = "sgemm" if "sgemm" in name else "hgemm" if "hgemm" in name else None
        if kind is None:
            continue
        v.sort()
        tail = [d for _, d in v[-TRACE_STEPS:]]
        out.append(f"| `{short(name)}` | {len(tail)} | {sum(tail) / len(tail) / 1e3:.1f} | "
                   f"{bench_line['per_kernel'][kind]['avg_ms'] * 1e3:.1f} |")
    out += ["", "The bench averages include the gap between an event and its kernel; rocprofv3 times "
                "the kernel alone. Both kernels are the NN (no transpose) instantiations; the first flag of "
                "the HGEMM kernel selects the input format (false: fp16)."]
    path = os.path.join(ROOT, "profiles", "kernel_trace_sgemm4096x4096x1024_hgemm4096cube.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(path)
    return 0


COUNTER_PASSES = (
    "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
    "SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR GRBM_GUI_ACTIVE",
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_WAIT_INST_LDS "
    "SQ_ACTIVE_INST_LDS SQ_LDS_ADDR_CONFLICT GRBM_GUI_ACTIVE",
    "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_DRAM_sum TCC_EA0_WRREQ_DRAM_sum",
)


def write_counters(csv_paths) -> int:
    """Per-launch means of rocprofv3 counters for the step's two kernels, with the
    derived figures the kernel design relies on (cycles per MFMA instruction, LDS bank
    conflicts), written as a markdown summary under profiles/."""
    import csv

    vals = {}          # kind -> counter -> list of per-dispatch values
    durs = {}          # kind -> list of dispatch durations (ns)
    names = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            kind = "sgemm" if "sgemm" in name else "hgemm" if "hgemm" in name else None
            if kind is None:
                continue
            names[kind] = name
            vals.setdefault(kind, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.setdefault(kind, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    mean = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}
    kinds = [k for k in ("sgemm", "hgemm") if k in mean]
    counters = sorted({c for k in kinds for c in mean[k]})
    cmds = "\n".join(
        f"cd /tmp && rocprofv3 --pmc {p} --output-format csv -d $OUT/counters{i} -o c -- "
        f"python3 $R/bench.py --no-cpu --no-extra --steps 3 --warmup 1" for i, p in enumerate(COUNTER_PASSES, 1))
    cmds += ("\npython3 $R/bench.py --write-counters " +
             " ".join(f"$OUT/counters{i}/c_counter_collection.csv" for i in range(1, len(COUNTER_PASSES) + 1)) +
             "   # R = repository root, OUT = an output directory")
    lines = ["# rocprofv3 counters per launch: bench step kernels (SGEMM 4096x4096x1024 fp32, "
             "HGEMM 4096^3 fp16->fp32)", "",
             "Commands (one MI355X; each pass is a run of its own):", "", "```", cmds, "```", "",
             "Mean over the dispatches of each kernel in the runs (the counters are summed over the "
             "whole device; SQ_LDS_* and SQ_*_CYCLES count in units of four cycles).", "",
             "| counter | " + " | ".join(kinds) + " |", "|---|" + "---|" * len(kinds)]
    for c in counters:
        lines.append(f"| {c} | " + " | ".join(f"{mean[k].get(c, float('nan')):.4g}" for k in kinds) + " |")
    lines += ["", "Derived:", ""]
    for k in kinds:
        m = mean[k]
        d = sum(durs[k]) / len(durs[k]) / 1e3
        short = names[k].replace("mi355gemm::(anonymous namespace)::", "").split("(")[0]
        parts = [f"- {k} (`{short}`, "
                 f"{d:.1f} us per profiled launch):"]
        if m.get("SQ_INSTS_MFMA"):
            parts.append(f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / m['SQ_INSTS_MFMA']:.1f} matrix-core cycles "
                         f"per MFMA instruction, {m['SQ_INSTS_MFMA']:.4g} MFMA instructions;")
        if m.get("SQ_LDS_IDX_ACTIVE"):
            parts.append(f"LDS bank conflicts {100 * m.get('SQ_LDS_BANK_CONFLICT', 0) / m['SQ_LDS_IDX_ACTIVE']:.2f}% "
                         f"of LDS-active cycles;")
        if m.get("TCC_HIT_sum") is not None and m.get("TCC_MISS_sum"):
            parts.append(f"L2 hit rate {100 * m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.1f}%;")
        if m.get("SQ_INSTS_MFMA") and m.get("SQ_INSTS_VALU") is not None:
            parts.append(f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f} VALU instructions (MFMA included) "
                         f"per MFMA.")
        lines.append(" ".join(parts))
    path = os.path.join(ROOT, "profiles", "counters_sgemm4096x4096x1024_hgemm4096cube.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)
    return 0


def write_traffic(fetch_csv: str, write_csv: str) -> int:
    """Per-launch HBM traffic of the step's kernels from FETCH_SIZE / WRITE_SIZE counter
    runs, each scaled by the ratio of known bytes to counted bytes for the calibration copy."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, value = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0
            kind = "sgemm" if "sgemm" in name else "hgemm" if "hgemm" in name else "copy"
            if kind == "copy" and value < COPY_BYTES / 8:
                continue   # other small kernels of the run (tensor fills), not the calibration copy
            vals.setdefault(kind, {}).setdefault(name, []).append(value)
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def mean(d, kind):
        (name, v), = d[kind].items()
        return name, sum(v) / len(v)

    copy_name, copy_f = mean(fetch, "copy")
    _, copy_w = mean(write, "copy")
    scale_f, scale_w = COPY_BYTES / copy_f, COPY_BYTES / copy_w
    workloads = {"sgemm": "SGEMM fp32 row-major 4096x4096x1024 alpha=1 beta=0",
                 "hgemm": "HGEMM fp16->fp32 row-major 4096x4096x4096 alpha=1 beta=0"}
    alg = {"sgemm": 4 * (4096 * 1024 * 2 + 4096 * 4096), "hgemm": 2 * (4096 * 4096 * 2) + 4 * 4096 * 4096}
    recs = {"copy_calibration": {"kernel": copy_name, "bytes": COPY_BYTES, "fetch_counted": copy_f,
                                 "write_counted": copy_w, "fetch_scale": scale_f, "write_scale": scale_w}}
    rows = []
    for kind in ("sgemm", "hgemm"):
        name, f = mean(fetch, kind)
        _, w = mean(write, kind)
        total = f * scale_f + w * scale_w
        recs[kind] = {"kernel": name, "workload": workloads[kind], "source_sha": source_digest(kind),
                      "fetch_bytes_per_launch": f * scale_f, "write_bytes_per_launch": w * scale_w,
                      "hbm_bytes_per_launch": total, "algorithmic_bytes": alg[kind]}
        rows.append(f"| {kind} | {workloads[kind]} | {f * scale_f / 1e6:.1f} | {w * scale_w / 1e6:.1f} | "
                    f"{total / 1e6:.1f} | {alg[kind] / 1e6:.1f} | {total / alg[kind]:.2f} |")
    cmd = ("cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/traffic_fetch -o t -- "
           "python3 $R/bench.py --no-cpu --no-extra --steps 3 --warmup 1 --copy-calibration\n"
           "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/traffic_write -o t -- "
           "python3 $R/bench.py --no-cpu --no-extra --steps 3 --warmup 1 --copy-calibration\n"
           "python3 $R/bench.py --write-traffic $OUT/traffic_fetch/t_counter_collection.csv "
           "$OUT/traffic_write/t_counter_collection.csv   # R = repository root, OUT = an output directory")
    text = ("# HBM traffic per launch: bench step kernels (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n"
            f"Commands (one MI355X):\n\n```\n{cmd}\n```\n\n"
            f"Calibration: a plain elementwise copy of {COPY_BYTES >> 20} MiB reads and writes {COPY_BYTES} bytes; "
            f"the counters read {copy_f:.0f} B fetched and {copy_w:.0f} B written, so fetch counts are scaled by "
            f"{scale_f:.4f} and write counts by {scale_w:.4f}.\n\n"
            "| kernel | workload | fetched (MB) | written (MB) | total (MB) | algorithmic (MB) | ratio |\n"
            "|---|---|---|---|---|---|---|\n" + "\n".join(rows) + "\n\n"
            "Machine-readable copy (bench.py reads it; a record whose source_sha no longer matches the kernel "
            "source is ignored):\n\n```json\n" + json.dumps(recs, indent=1) + "\n```\n")
    with open(TRAFFIC_FILE, "w") as f:
        f.write(text)
    print(text)
    return 0


def time_calls(fn, torch, stream, warmup=20, reps=30, graph_calls=20):
    """Seconds per call of fn(s), which enqueues one library call on stream s.

    Returns (median, min) over `reps` calls, each between its own pair of events on
    `stream` (so a launch gap before the kernel counts), and the median over five
    replays of one HIP graph holding `graph_calls` calls back to back, divided by
    `graph_calls` (kernel time without launch gaps: what matters for kernels of a
    few microseconds)."""
    for _ in range(warmup):
        fn(stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn(stream)
        b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for _ in range(graph_calls):
            fn(side)
    g.replay()
    torch.cuda.synchronize()
    tg = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        tg.append(a.elapsed_time(b) * 1e-3 / graph_calls)
    del g
    return ts[len(ts) // 2], ts[0], sorted(tg)[2]


def rates(med, graph, flop, peak):
    """Extra-workload record: per-call median (launch-inclusive) and back-to-back graph time."""
    return {"median_ms": med * 1e3, "tflops": flop / med / 1e12, "frac_of_peak": flop / med / 1e12 / peak,
            "graph_ms_per_call": graph * 1e3, "graph_tflops": flop / graph / 1e12}


def run_extra(dg, si, np, torch, dev, stream):
    out = {}

    def up(buf):
        return torch.from_numpy(np.ascontiguousarray(buf)).to(dev)

    def sg(M, N, K, alpha, beta, name):
        p = si.gemm_problem(M, N, K, seed=42, with_c=beta != 0)
        A, B = up(p["A"]), up(p["B"])
        C = up(p["C"]) if beta != 0 else torch.empty(M * N, dtype=torch.float32, device=dev)
        med, _, gr = time_calls(lambda s: dg.gemm_f32(M, N, K, alpha, A, K, B, N, beta, C, N, s), torch, stream)
        out[name] = rates(med, gr, 2.0 * M * N * K, PEAK_F32_TFLOPS)

    sg(512, 512, 512, 1.0, 0.0, "sgemm_512^3")
    sg(1001, 777, 513, 1.5, -0.5, "sgemm_1001x777x513_a1.5_b-0.5")
    sg(1024, 1024, 512, 1.5, -0.5, "sgemm_1024x1024x512_a1.5_b-0.5")
    for n in (1024, 2048, 8192):
        sg(n, n, 1024, 1.0, 0.0, f"sgemm_{n}x{n}x1024")

    p = si.gemm_problem(2048, 2048, 2048, in_dtype=np.float16, seed=42, with_c=False)
    A, B = up(p["A"]), up(p["B"])
    C = torch.empty(2048 * 2048, dtype=torch.float32, device=dev)
    med, _, gr = time_calls(lambda s: dg.gemm_f16_f32acc(2048, 2048, 2048, 1.0, A, 2048, B, 2048, 0.0, C, 2048, s),
                            torch, stream)
    out["hgemm_2048^3"] = rates(med, gr, 2.0 * 2048 ** 3, PEAK_F16_TFLOPS)

    # one GPU's share of the step when 8 GPUs split C by rows (512 of the 4096 rows)
    for kind, (M, N, K) in (("sgemm", (512, 4096, 1024)), ("hgemm", (512, 4096, 4096))):
        dt = torch.float32 if kind == "sgemm" else torch.float16
        A = torch.empty(M * K, dtype=dt, device=dev).uniform_(-1, 1)
        B = torch.empty(K * N, dtype=dt, device=dev).uniform_(-1, 1)
        C = torch.empty(M * N, dtype=torch.float32, device=dev)
        fn = dg.gemm_f32 if kind == "sgemm" else dg.gemm_f16_f32acc
        med, _, gr = time_calls(lambda s: fn(M, N, K, 1.0, A, K, B, N, 0.0, C, N, s), torch, stream)
        peak = PEAK_F32_TFLOPS if kind == "sgemm" else PEAK_F16_TFLOPS
        out[f"{kind}_row_share_1of8_{M}x{N}x{K}"] = rates(med, gr, 2.0 * M * N * K, peak)

    # bfloat16 inputs (the same kernels with the bf16 matrix-core op)
    for n in (2048, 4096):
        A = torch.empty(n * n, dtype=torch.bfloat16, device=dev).uniform_(-1, 1)
        B = torch.empty(n * n, dtype=torch.bfloat16, device=dev).uniform_(-1, 1)
        C = torch.empty(n * n, dtype=torch.float32, device=dev)
        med, _, gr = time_calls(lambda s: dg.gemm_bf16_f32acc(n, n, n, 1.0, A, n, B, n, 0.0, C, n, s), torch, stream)
        out[f"bf16gemm_{n}^3"] = rates(med, gr, 2.0 * n ** 3, PEAK_BF16_TFLOPS)

    # ragged shapes (M, N not multiples of the tile, K not of the slice): the masked
    # direct-to-LDS kernels
    for kind, (M, N, K) in (("sgemm", (4000, 4000, 1000)), ("hgemm", (4000, 4000, 4000))):
        dt = torch.float32 if kind == "sgemm" else torch.float16
        A = torch.empty(M * K, dtype=dt, device=dev).uniform_(-1, 1)
        B = torch.empty(K * N, dtype=dt, device=dev).uniform_(-1, 1)
        C = torch.empty(M * N, dtype=torch.float32, device=dev)
        fn = dg.gemm_f32 if kind == "sgemm" else dg.gemm_f16_f32acc
        med, _, gr = time_calls(lambda s: fn(M, N, K, 1.0, A, K, B, N, 0.0, C, N, s), torch, stream)
        peak = PEAK_F32_TFLOPS if kind == "sgemm" else PEAK_F16_TFLOPS
        out[f"{kind}_ragged_{M}x{N}x{K}"] = rates(med, gr, 2.0 * M * N * K, peak)

    # op(A)op(B): the bench shapes with A stored K x M and/or B stored N x K
    for tA, tB in ((0, 1), (1, 0), (1, 1)):
        tag = ("T" if tA else "N") + ("T" if tB else "N")
        for kind, (M, N, K) in (("sgemm", (4096, 4096, 1024)), ("hgemm", (4096, 4096, 4096))):
            dt = torch.float32 if kind == "sgemm" else torch.float16
            A = torch.empty(M * K, dtype=dt, device=dev).uniform_(-1, 1)
            B = torch.empty(K * N, dtype=dt, device=dev).uniform_(-1, 1)
            C = torch.empty(M * N, dtype=torch.float32, device=dev)
            lda, ldb = (M if tA else K), (K if tB else N)
            fn = dg.gemm_f32_ex if kind == "sgemm" else dg.gemm_f16_f32acc_ex
            med, _, gr = time_calls(lambda s: fn(tA, tB, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, N, s), torch, stream)
            peak = PEAK_F32_TFLOPS if kind == "sgemm" else PEAK_F16_TFLOPS
            out[f"{kind}_{tag}_{M}x{N}x{K}"] = rates(med, gr, 2.0 * M * N * K, peak)

    # 16 x 1024^3 batched, beta = 1 (C is read and written: HBM-bound, ridge below the fp16 peak)
    nb, n = 16, 1024
    A = torch.empty(nb * n * n, dtype=torch.float16, device=dev).uniform_(-1, 1)
    B = torch.empty(nb * n * n, dtype=torch.float16, device=dev).uniform_(-1, 1)
    C = torch.empty(nb * n * n, dtype=torch.float32, device=dev).uniform_(-1, 1)
    med, _, gr = time_calls(lambda s: dg.gemm_batched_f16_f32acc(n, n, n, 1.0, A, n, n * n, B, n, n * n, 1.0, C, n,
                                                                 n * n, nb, s), torch, stream)
    fl = 2.0 * nb * n ** 3
    bytes_alg = nb * n * n * (2 + 2 + 4 + 4)
    out["batched_hgemm_16x1024^3_b1"] = dict(rates(med, gr, fl, PEAK_F16_TFLOPS),
                                             hbm_roofline_tflops=min(PEAK_F16_TFLOPS, fl / bytes_alg * PEAK_HBM_GBS / 1e3),
                                             warm_buffers=True)
    # cold: three operand sets (384 MB, more than the 256 MB last-level cache) used in turn,
    # so each call finds its inputs in HBM
    sets = [(torch.empty(nb * n * n, dtype=torch.float16, device=dev).uniform_(-1, 1),
             torch.empty(nb * n * n, dtype=torch.float16, device=dev).uniform_(-1, 1),
             torch.empty(nb * n * n, dtype=torch.float32, device=dev).uniform_(-1, 1)) for _ in range(3)]
    turn = [0]

    def cold_call(s):
        a, b, c = sets[turn[0] % 3]
        turn[0] += 1
        dg.gemm_batched_f16_f32acc(n, n, n, 1.0, a, n, n * n, b, n, n * n, 1.0, c, n, n * n, nb, s)

    med, _, gr = time_calls(cold_call, torch, stream, graph_calls=21)
    hbm_roof = min(PEAK_F16_TFLOPS, fl / bytes_alg * PEAK_HBM_GBS / 1e3)
    out["batched_hgemm_16x1024^3_b1_cold"] = dict(rates(med, gr, fl, PEAK_F16_TFLOPS), hbm_roofline_tflops=hbm_roof,
                                                  frac_of_hbm_roofline=fl / med / 1e12 / hbm_roof,
                                                  warm_buffers=False, operand_sets=3)
    del sets
    return out


def cpu_baseline(si, np, ps, ph, budget_s):
    """The oracle, as it stands, on row blocks of both workloads until the time budget is spent."""
    import oracle

    threads = oracle.default_threads()
    flops = 0.0
    rows_s = rows_h = 0
    t0 = time.perf_counter()
    block = 128
    while time.perf_counter() - t0 < budget_s and (rows_s < 4096 or rows_h < 4096):
        if rows_s < 4096:
            rows = np.arange(rows_s, rows_s + block, dtype=np.int32)
            oracle.gemm_ref(4096, 4096, 1024, 1.0, ps["A"], 1024, ps["B"], 4096, 0.0, None, 4096,
                            rows=rows, threads=threads)
            rows_s += block
            flops += 2.0 * block * 4096 * 1024
        if rows_h < 4096 and time.perf_counter() - t0 < budget_s:
            rows = np.arange(rows_h, rows_h + block, dtype=np.int32)
            oracle.gemm_ref(4096, 4096, 4096, 1.0, ph["A"], 4096, ph["B"], 4096, 0.0, None, 4096,
                            rows=rows, threads=threads)
            rows_h += block
            flops += 2.0 * block * 4096 * 4096
    dt = time.perf_counter() - t0
    # the same loop on one thread, over a short sample of SGEMM rows
    t1 = time.perf_counter()
    one_rows = 128
    oracle.gemm_ref(4096, 4096, 1024, 1.0, ps["A"], 1024, ps["B"], 4096, 0.0, None, 4096,
                    rows=np.arange(one_rows, dtype=np.int32), threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"first {rows_s} rows of the SGEMM 4096x4096x1024 and first {rows_h} rows of the "
                      f"HGEMM 4096^3 (fp64 triple loop), {dt:.1f} s",
            "single_thread": {"value": 2.0 * one_rows * 4096 * 1024 / dt1 / 1e12, "unit": "TFLOPS",
                              "sample": f"first {one_rows} rows of the SGEMM 4096x4096x1024, {dt1:.2f} s"}}


if __name__ == "__main__":
    sys.exit(main())
