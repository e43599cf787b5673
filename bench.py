"""Benchmark of the row-major GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

One step is one SGEMM of 4096x4096x1024 (fp32) followed by one HGEMM of
4096x4096x4096 (fp16 inputs, fp32 accumulation and output), alpha = 1 and
beta = 0, on seeded uniform[-1,1) inputs already resident in HBM.  The value is
the step's throughput, (2*4096*4096*1024 + 2*4096^3) / step time, in TFLOPS;
the per-kernel TFLOPS and fraction of the MI355X peak for its dtype are
reported beside it, with the roofline of the dominant (longest) kernel taken
from HIP events recorded on the stream the kernels run on.  The CPU oracle is
timed on the same workload as a baseline, and on every other benchmark
configuration under "cpu_per_config".

Clock: the shader clock takes some tens of milliseconds of load to leave its
idle state.  Before the warm-up steps the step runs back to back for
--settle-ms (untimed) while the clock is sampled; "clock" reports the samples
(idle, under that load, and right after the timed steps) and where they were
read.

The other benchmark configurations (SGEMM 512^3; the 1001x777x513 and
1024x1024x512 SGEMMs with alpha = 1.5, beta = -0.5 and with alpha = 1,
beta = 0; the M = N sweep at K = 1024 from 128 to 16384; HGEMM 2048^3 and
4096^3; 16 batched 1024^3 HGEMMs with beta = 1, warm and cold), one GPU's
share of each step shape under an 8-way row split, bf16 inputs, two ragged
shapes and the transposed storage combinations are timed after the main run
and reported under "extra" (not part of the value).

    python bench.py --profile NAME [--steps K] [--warmup W] [--copy-calibration]

runs only configuration NAME ("step" or a key of "extra") K times after W
untimed calls and prints one short line: the command rocprofv3 wraps to collect
a configuration's counters.  --write-counters / --write-traffic /
--write-trace turn such runs' CSV files into the summaries under profiles/.

Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS (2MNK/t) + % of dtype peak: SGEMM 4096x4096x1024, HGEMM 4096^3"
# MI355X peaks: 256 CUs x 2.4 GHz; fp32 matrix/vector 256 flop/clk/CU, fp16 dense MFMA 4096 flop/clk/CU.
PEAK_F32_TFLOPS = 157.3
PEAK_F16_TFLOPS = 2516.6
PEAK_BF16_TFLOPS = 2516.6   # bf16 dense MFMA runs at the fp16 rate
PEAK_HBM_GBS = 8000.0
PEAKS = {"f32": PEAK_F32_TFLOPS, "f16": PEAK_F16_TFLOPS, "bf16": PEAK_BF16_TFLOPS}
_CSRC = "dense_gemm_optimisation_f32_amd/csrc/"
# the files whose code makes up each kernel (its source and the headers it includes)
KERNEL_SOURCES = {
    "sgemm": [_CSRC + f for f in ("sgemm_mfma.hip", "epilogue.h", "tile_order.h", "gemm_internal.h")],
    "hgemm": [_CSRC + f for f in ("hgemm_mfma.hip", "epilogue.h", "tile_order.h", "gemm_internal.h")],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
COPY_BYTES = 256 << 20   # size of the calibration copy (read and written)
STEP_WORKLOADS = {"sgemm": "SGEMM fp32 row-major 4096x4096x1024 alpha=1 beta=0",
                  "hgemm": "HGEMM fp16->fp32 row-major 4096x4096x4096 alpha=1 beta=0"}


def source_digest(kind: str) -> str:
    """Digest of a kernel's code: its files with comments and whitespace removed,
    so that a counter record stays valid across comment-only edits."""
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


def measured_traffic(key: str, kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when it is missing or was taken on a different version of the kernel source."""
    try:
        rec = _traffic_records()[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_digest(kind) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- configurations
def extra_configs():
    """The benchmark configurations timed besides the step, in order.  Each is one
    library call: kind (f32, f16, bf16), shape, alpha/beta, batch, storage flags."""
    out = []

    def add(name, kind, M, N, K, alpha=1.0, beta=0.0, batch=1, tA=0, tB=0, cold=False):
        out.append(dict(name=name, kind=kind, M=M, N=N, K=K, alpha=alpha, beta=beta, batch=batch,
                        tA=tA, tB=tB, cold=cold))

    # configuration 1
    add("sgemm_512^3", "f32", 512, 512, 512)
    # configuration 2: the non-multiple and the regular shape, with the alpha/beta
    # epilogue and at alpha = 1, beta = 0
    for M, N, K in ((1001, 777, 513), (1024, 1024, 512)):
        add(f"sgemm_{M}x{N}x{K}_a1.5_b-0.5", "f32", M, N, K, 1.5, -0.5)
        add(f"sgemm_{M}x{N}x{K}", "f32", M, N, K)
    # configuration 3: the M = N sweep at K = 1024 (4096 is the step's SGEMM, here alone)
    for n in (128, 256, 512, 1024, 2048, 4096, 8192, 16384):
        add(f"sgemm_{n}x{n}x1024", "f32", n, n, 1024)
    # configuration 4 (4096^3 is the step's HGEMM, here alone)
    for n in (2048, 4096):
        add(f"hgemm_{n}^3", "f16", n, n, n)
    # configuration 5: warm (the same buffers every call) and cold (operand sets
    # larger than the last-level cache used in turn)
    add("batched_hgemm_16x1024^3_b1", "f16", 1024, 1024, 1024, 1.0, 1.0, batch=16)
    add("batched_hgemm_16x1024^3_b1_cold", "f16", 1024, 1024, 1024, 1.0, 1.0, batch=16, cold=True)
    # few tiles and a long K: the HGEMM splits each tile's K range over workgroups
    add("hgemm_splitk_512x512x8192", "f16", 512, 512, 8192)
    add("hgemm_splitk_1024x1024x8192", "f16", 1024, 1024, 8192)
    # one GPU's share of each step shape when 8 GPUs split C by rows
    add("sgemm_row_share_1of8_512x4096x1024", "f32", 512, 4096, 1024)
    add("hgemm_row_share_1of8_512x4096x4096", "f16", 512, 4096, 4096)
    # bfloat16 inputs (the same kernels with the bf16 matrix-core op)
    for n in (2048, 4096):
        add(f"bf16gemm_{n}^3", "bf16", n, n, n)
    # ragged shapes: the masked direct-to-LDS kernels
    add("sgemm_ragged_4000x4000x1000", "f32", 4000, 4000, 1000)
    add("hgemm_ragged_4000x4000x4000", "f16", 4000, 4000, 4000)
    # op(A)op(B): the step shapes with A stored K x M and/or B stored N x K
    for tA, tB in ((0, 1), (1, 0), (1, 1)):
        tag = ("T" if tA else "N") + ("T" if tB else "N")
        add(f"sgemm_{tag}_4096x4096x1024", "f32", 4096, 4096, 1024, tA=tA, tB=tB)
        add(f"hgemm_{tag}_4096x4096x4096", "f16", 4096, 4096, 4096, tA=tA, tB=tB)
    return out


def config_bytes(c):
    """Algorithmic bytes of one call: A and B read once, C written once and read when beta != 0."""
    ein = 4 if c["kind"] == "f32" else 2
    per = ein * (c["M"] * c["K"] + c["K"] * c["N"]) + 4 * c["M"] * c["N"] * (2 if c["beta"] != 0 else 1)
    return per * c["batch"]


def config_flop(c):
    return 2.0 * c["M"] * c["N"] * c["K"] * c["batch"]


class ConfigRunner:
    """Seeded operands of one configuration resident on the device, and a closure
    that enqueues the library call on a given stream."""

    def __init__(self, c, dg, si, np, torch, dev, sets=1):
        self.c = c
        M, N, K, nb = c["M"], c["N"], c["K"], c["batch"]
        in_dtype = {"f32": np.float32, "f16": np.float16, "bf16": "bf16"}[c["kind"]]
        a_rows, a_cols = (K, M) if c["tA"] else (M, K)
        b_rows, b_cols = (N, K) if c["tB"] else (K, N)
        self.lda, self.ldb, self.ldc = a_cols, b_cols, N

        def up(buf):
            buf = np.ascontiguousarray(buf)
            if buf.dtype == np.uint16:
                return torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(buf).to(dev)

        self.sets = []
        for s in range(sets):
            probs = [si.gemm_problem(M, N, K, in_dtype=in_dtype, seed=42 + 1000 * s, batch=b,
                                     with_c=c["beta"] != 0, transA=bool(c["tA"]), transB=bool(c["tB"]))
                     for b in range(nb)]
            A = up(np.concatenate([p["A"] for p in probs]))
            B = up(np.concatenate([p["B"] for p in probs]))
            if c["beta"] != 0:
                C = up(np.concatenate([p["C"] for p in probs]))
            else:
                C = torch.empty(nb * M * N, dtype=torch.float32, device=dev)
            self.sets.append((A, B, C))
            del probs
        self.turn = 0
        self.dg = dg

    def __call__(self, stream):
        c, dg = self.c, self.dg
        A, B, C = self.sets[self.turn % len(self.sets)]
        self.turn += 1
        M, N, K, nb = c["M"], c["N"], c["K"], c["batch"]
        if nb > 1:
            fn = dg.gemm_batched_bf16_f32acc_ex if c["kind"] == "bf16" else dg.gemm_batched_f16_f32acc_ex
            fn(c["tA"], c["tB"], M, N, K, c["alpha"], A, self.lda, M * K, B, self.ldb, K * N, c["beta"], C,
               self.ldc, M * N, nb, stream)
            return
        fn = {"f32": dg.gemm_f32_ex, "f16": dg.gemm_f16_f32acc_ex, "bf16": dg.gemm_bf16_f32acc_ex}[c["kind"]]
        fn(c["tA"], c["tB"], M, N, K, c["alpha"], A, self.lda, B, self.ldb, c["beta"], C, self.ldc, stream)


# ---------------------------------------------------------------- clock
def _sysfs_sclk():
    """Current shader clock (MHz) of each GPU the sysfs DPM tables show: the level
    marked '*' in pp_dpm_sclk."""
    vals = []
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if "*" in line:
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    if m:
                        vals.append(int(m.group(1)))
        except OSError:
            continue
    return vals


def _smi_sclk():
    """Shader clock (MHz) as rocm-smi reports it (the current sclk level)."""
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return []
    vals = []
    for line in out.splitlines():
        if "sclk" in line.lower():
            m = re.search(r"\((\d+)\s*[Mm][Hh]z\)", line)
            if m:
                vals.append(int(m.group(1)))
    return vals


def read_sclk():
    """(MHz values, source) of the shader clock, from sysfs when readable, else rocm-smi."""
    v = _sysfs_sclk()
    if v:
        return v, "sysfs pp_dpm_sclk"
    v = _smi_sclk()
    return v, ("rocm-smi --showclocks" if v else "unavailable")


class ClockSampler:
    """Samples the shader clock in a background thread until stopped."""

    def __init__(self, period_s=0.02):
        self.period = period_s
        self.samples = []
        self.source = None
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            v, src = read_sclk()
            if v:
                self.samples.append(v[0])
                self.source = src
            self._stop.wait(self.period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=30)


# ---------------------------------------------------------------- timing helpers
def time_calls(fn, torch, stream, warmup=20, reps=30, graph_calls=20, warm_s=0.1):
    """Seconds per call of fn(s), which enqueues one library call on stream s.

    Warm-up: at least `warmup` calls and `warm_s` seconds of back-to-back calls, so
    the shader clock has left its idle state (the host-side input generation before
    each configuration leaves the GPU idle for long enough to drop it).
    Returns (median, min) over `reps` calls, each between its own pair of events on
    `stream` (so a launch gap before the kernel counts), and the median over five
    replays of one HIP graph holding `graph_calls` calls back to back, divided by
    `graph_calls` (kernel time without launch gaps: what matters for kernels of a
    few microseconds)."""
    t_end = time.perf_counter() + warm_s
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        for _ in range(10):
            fn(stream)
        n += 10
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
    # one call on the capture stream first: a K split keeps its scratch per stream
    # and cannot allocate it during capture, so this makes the graph record the
    # same plan as the calls timed above
    fn(side)
    torch.cuda.synchronize()
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


# ---------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back steps before the warm-up, while the clock is sampled")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baselines")
    ap.add_argument("--no-extra", action="store_true", help="skip the other configurations")
    ap.add_argument("--only", nargs="+", metavar="NAME", help="time only these extra configurations")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle time budget for the step")
    ap.add_argument("--profile", metavar="NAME",
                    help="run only configuration NAME ('step' or an extra key) --steps times after --warmup calls")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy three times (counter calibration)")
    ap.add_argument("--write-traffic", nargs=3, metavar=("NAME", "FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a "
                         "--profile NAME --copy-calibration run into a record of profiles/hbm_traffic.md")
    ap.add_argument("--write-trace", nargs=3, metavar=("STATS_CSV", "TRACE_CSV", "BENCH_LOG"),
                    help="turn a rocprofv3 --kernel-trace --stats run of this script into "
                         "profiles/kernel_trace_sgemm4096x4096x1024_hgemm4096cube.md; uses no GPU")
    ap.add_argument("--write-counters", nargs="+", metavar=("NAME", "CSV"),
                    help="turn rocprofv3 counter_collection.csv files of a --profile NAME run into "
                         "profiles/counters_NAME.md; uses no GPU")
    ap.add_argument("--write-resources", action="store_true",
                    help="write the compiler's register, scratch, LDS and occupancy figures of the "
                         "profiled kernels to profiles/resources.md (runs hipcc; uses no GPU)")
    args = ap.parse_args()
    if args.write_resources:
        return write_resources()
    if args.write_traffic:
        return write_traffic(*args.write_traffic)
    if args.write_counters:
        return write_counters(args.write_counters[0], args.write_counters[1:])
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

    if args.profile and args.profile != "step":
        return profile_config(args, dg, si, np, torch, dev, stream)

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
        copy_calibration(torch, dev)

    def sgemm():
        dg.gemm_f32(Ms, Ns, Ks, 1.0, sA, Ks, sB, Ns, 0.0, sC, Ns, stream)

    def hgemm():
        dg.gemm_f16_f32acc(Mh, Nh, Kh, 1.0, hA, Kh, hB, Nh, 0.0, hC, Nh, stream)

    if args.profile == "step":
        for _ in range(args.warmup):
            sgemm()
            hgemm()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            sgemm()
            hgemm()
        torch.cuda.synchronize()
        print(f"profiled step: {args.steps} steps after {args.warmup}", flush=True)
        return 0

    # ---- clock: idle, then under back-to-back steps (untimed), then the warm-up
    idle_mhz, clock_src = read_sclk()
    settle_steps = 0
    with ClockSampler() as sampler:
        t_end = time.perf_counter() + args.settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(20):
                sgemm()
                hgemm()
            settle_steps += 20
            torch.cuda.synchronize()
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
    after_mhz, _ = read_sclk()

    t_s = [e[0].elapsed_time(e[1]) * 1e-3 for e in ev]
    t_h = [e[1].elapsed_time(e[2]) * 1e-3 for e in ev]
    flop_s = 2.0 * Ms * Ns * Ks
    flop_h = 2.0 * Mh * Nh * Kh
    step_s = wall / args.steps
    value = (flop_s + flop_h) / step_s / 1e12

    def kernel_record(ts, flop, peak, workload, bytes_alg):
        avg = statistics.fmean(ts)
        return {
            "workload": workload,
            "avg_ms": avg * 1e3, "median_ms": statistics.median(ts) * 1e3, "min_ms": min(ts) * 1e3,
            "tflops": flop / avg / 1e12, "peak_tflops": peak, "frac_of_peak": flop / avg / 1e12 / peak,
            "algorithmic_flop": flop, "algorithmic_bytes": bytes_alg,
        }

    bytes_s = 4 * (Ms * Ks + Ks * Ns + Ms * Ns)
    bytes_h = 2 * (Mh * Kh + Kh * Nh) + 4 * Mh * Nh
    per_kernel = {
        "sgemm": kernel_record(t_s, flop_s, PEAK_F32_TFLOPS, STEP_WORKLOADS["sgemm"], bytes_s),
        "hgemm": kernel_record(t_h, flop_h, PEAK_F16_TFLOPS, STEP_WORKLOADS["hgemm"], bytes_h),
    }
    dom = max(per_kernel, key=lambda k: per_kernel[k]["avg_ms"])
    dk = per_kernel[dom]
    roofline = {
        "kernel": dom, "bound": "mfma", "achieved": dk["tflops"], "peak": dk["peak_tflops"],
        "unit": "TFLOP/s", "frac": dk["frac_of_peak"], "traffic": measured_traffic(dom, dom, dk["workload"]),
        "algorithmic_flop_per_launch": dk["algorithmic_flop"],
    }
    other = "hgemm" if dom == "sgemm" else "sgemm"
    ok = per_kernel[other]
    roofline_other = {
        "kernel": other, "bound": "mfma", "achieved": ok["tflops"], "peak": ok["peak_tflops"],
        "unit": "TFLOP/s", "frac": ok["frac_of_peak"], "traffic": measured_traffic(other, other, ok["workload"]),
    }
    s = sampler.samples
    clock = {"source": sampler.source or clock_src, "idle_mhz": idle_mhz[:1] or None,
             "settle_ms": args.settle_ms, "settle_steps": settle_steps,
             "under_step_load_mhz": {"samples": len(s), "min": min(s) if s else None,
                                     "median": statistics.median(s) if s else None,
                                     "max": max(s) if s else None},
             "after_timed_steps_mhz": after_mhz[:1] or None}

    extra = {}
    if not args.no_extra:
        extra = run_extra(dg, si, np, torch, dev, stream, args.only)

    cpu = cpu_per = None
    if not args.no_cpu:
        cpu = cpu_baseline(si, np, ps, ph, args.cpu_seconds)
        if not args.only:
            cpu_per = cpu_per_config(si, np)

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
        "clock": clock,
        "extra": extra,
        "cpu_per_config": cpu_per,
    }
    print(json.dumps(line), flush=True)
    return 0


def copy_calibration(torch, dev):
    """A plain 256 MiB elementwise copy, three times: the reference dispatch whose
    FETCH_SIZE / WRITE_SIZE counts scale the kernels' counts to bytes."""
    # uninitialised buffers: no fill kernel joins the counted dispatches
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)   # reads and writes COPY_BYTES
    torch.cuda.synchronize()
    del src, dst


def profile_config(args, dg, si, np, torch, dev, stream):
    """--profile NAME: only configuration NAME, --steps calls after --warmup calls."""
    cfg = {c["name"]: c for c in extra_configs()}.get(args.profile)
    if cfg is None:
        print(f"unknown configuration {args.profile!r}; choose 'step' or one of: "
              + ", ".join(c["name"] for c in extra_configs()), file=sys.stderr)
        return 2
    run = ConfigRunner(cfg, dg, si, np, torch, dev, sets=3 if cfg["cold"] else 1)
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(torch, dev)
    # at least --warmup calls and 100 ms of back-to-back calls (the clock leaves its idle state)
    n, t_end = 0, time.perf_counter() + 0.1
    while n < args.warmup or time.perf_counter() < t_end:
        run(stream)
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        run(stream)
    torch.cuda.synchronize()
    print(f"profiled {args.profile}: {args.steps} calls after {n}", flush=True)
    return 0


def run_extra(dg, si, np, torch, dev, stream, only=None):
    out = {}
    for c in extra_configs():
        if only and c["name"] not in only:
            continue
        run = ConfigRunner(c, dg, si, np, torch, dev, sets=3 if c["cold"] else 1)
        # cold: 21 graph calls over three operand sets (each set ~67 MB of A and B
        # plus 67 MB of C: 403 MB in all, more than the 256 MB last-level cache)
        med, _, gr = time_calls(run, torch, stream, graph_calls=21 if c["cold"] else 20)
        fl = config_flop(c)
        rec = rates(med, gr, fl, PEAKS[c["kind"]])
        if c["batch"] > 1:
            roof = min(PEAKS[c["kind"]], fl / config_bytes(c) * PEAK_HBM_GBS / 1e3)
            rec.update(hbm_roofline_tflops=roof, frac_of_hbm_roofline=fl / med / 1e12 / roof,
                       graph_frac_of_hbm_roofline=fl / gr / 1e12 / roof,
                       warm_buffers=not c["cold"], operand_sets=len(run.sets))
        out[c["name"]] = rec
        del run
        torch.cuda.empty_cache()
    return out


def cpu_baseline(si, np, ps, ph, budget_s):
    """The oracle, as it stands, on row blocks of both step workloads until the time budget is spent."""
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


# the benchmark configurations the oracle is timed on (the others repeat one of
# these shapes with other alpha/beta, storage flags or cache state)
CPU_CONFIGS = ("sgemm_512^3", "sgemm_1001x777x513_a1.5_b-0.5", "sgemm_1024x1024x512_a1.5_b-0.5",
               *(f"sgemm_{n}x{n}x1024" for n in (128, 256, 512, 1024, 2048, 4096, 8192, 16384)),
               "hgemm_2048^3", "hgemm_4096^3", "batched_hgemm_16x1024^3_b1")


def cpu_per_config(si, np):
    """The oracle on each benchmark configuration: the whole C up to 4096 rows (all
    16 members of the batch), 64 seeded rows of the 8192 and 16384 sweep points."""
    import oracle

    threads = oracle.default_threads()
    out = {}
    for c in extra_configs():
        if c["name"] not in CPU_CONFIGS:
            continue   # the same arithmetic as a configuration that is timed
        M, N, K, nb = c["M"], c["N"], c["K"], c["batch"]
        in_dtype = np.float16 if c["kind"] == "f16" else np.float32
        rows = si.sample_rows(42, M, 64) if M > 4096 else None
        n_rows = M if rows is None else len(rows)
        dt = 0.0
        for b in range(nb):
            p = si.gemm_problem(M, N, K, in_dtype=in_dtype, seed=42, batch=b, with_c=c["beta"] != 0)
            t0 = time.perf_counter()
            oracle.gemm_ref(M, N, K, c["alpha"], p["A"], p["lda"], p["B"], p["ldb"], c["beta"], p["C"], p["ldc"],
                            rows=rows, threads=threads)
            dt += time.perf_counter() - t0
        out[c["name"]] = {"gflops": 2.0 * n_rows * N * K * nb / dt / 1e9, "seconds": dt, "cores": threads,
                          "rows": "all" if rows is None else f"{n_rows} seeded rows of {M}"}
    return out


# ---------------------------------------------------------------- profile summaries
TRACE_STEPS, TRACE_WARMUP = 50, 20


def _short(n):
    return n.replace("mi355gemm::(anonymous namespace)::", "").split("(")[0]


def write_trace(stats_csv: str, trace_csv: str, bench_log: str) -> int:
    """Kernel-trace summary of a profiled run of this script: rocprofv3's statistics over
    all launches, the same over the timed launches only (the last TRACE_STEPS of each
    kernel), and the bench line's own HIP-event averages for comparison."""
    import csv

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
           "All launches (clock-settling steps and warm-up included):", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
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
        out.append(f"| `{_short(name)}` | {len(tail)} | {sum(tail) / len(tail) / 1e3:.1f} | "
                   f"{bench_line['per_kernel'][kind]['avg_ms'] * 1e3:.1f} |")
    ck = bench_line.get("clock") or {}
    out += ["", f"Shader clock ({ck.get('source')}): idle {ck.get('idle_mhz')} MHz, under back-to-back steps "
                f"{ck.get('under_step_load_mhz')}, right after the timed steps {ck.get('after_timed_steps_mhz')} MHz.",
            "", "The bench averages include the gap between an event and its kernel; rocprofv3 times "
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
    "TA_BUSY_avr TA_BUSY_max TA_FLAT_READ_LDS_WAVEFRONTS_sum TD_TD_BUSY_sum TD_TC_STALL_sum GRBM_GUI_ACTIVE",
)


def _slug(name: str) -> str:
    return re.sub(r"[^A-Za-z0-9_.-]", "", name.replace("^3", "cube").replace("^", ""))


def write_counters(name: str, csv_paths) -> int:
    """Per-launch means of rocprofv3 counters for the library's kernels in --profile NAME
    runs, with the derived figures the kernel design relies on (cycles per MFMA
    instruction, VALU instructions per MFMA, LDS bank conflicts, L2 hit rate), written as
    a markdown summary profiles/counters_NAME.md."""
    import csv

    vals, durs = {}, {}   # kernel -> counter -> values; kernel -> durations (ns)
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            kname = r["Kernel_Name"]
            if "gemm" not in kname:
                continue
            k = _short(kname) + ("<" + kname.split("<", 1)[1].split(">(")[0] + ">" if "<" in kname else "")
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    mean = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}
    kernels = sorted(mean)
    counters = sorted({c for k in kernels for c in mean[k]})
    what = "step" if name == "step" else name
    cmds = "\n".join(
        f"cd /tmp && timeout -s KILL 120 rocprofv3 --pmc {p} --output-format csv -d $OUT/counters{i} -o c -- "
        f"python3 $R/bench.py --profile {what} --steps 3 --warmup 1" for i, p in enumerate(COUNTER_PASSES, 1))
    cmds += (f"\npython3 $R/bench.py --write-counters {what} " +
             " ".join(f"$OUT/counters{i}/c_counter_collection.csv" for i in range(1, len(COUNTER_PASSES) + 1)) +
             "   # R = repository root, OUT = an output directory")
    title = ("bench step kernels (SGEMM 4096x4096x1024 fp32, HGEMM 4096^3 fp16->fp32)" if name == "step"
             else f"configuration {name}")
    lines = [f"# rocprofv3 counters per launch: {title}", "",
             "Commands (one MI355X; each pass is a run of its own):", "", "```", cmds, "```", "",
             "Mean over the dispatches of each kernel in the runs (each run warms the clock with about 100 ms of "
             "calls first, so most dispatches are those). Counters are summed over the whole device: "
             "SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs in cycles, SQ_WAVE_CYCLES and SQ_WAIT_* over the waves "
             "in units of four cycles, GRBM_GUI_ACTIVE over the 8 XCDs.", ""]
    for j, k in enumerate(kernels):
        lines.append(f"- kernel {j}: `{k}`")
    lines += ["", "| counter | " + " | ".join(f"kernel {j}" for j in range(len(kernels))) + " |",
              "|---|" + "---|" * len(kernels)]
    for c in counters:
        lines.append(f"| {c} | " + " | ".join(f"{mean[k].get(c, float('nan')):.4g}" for k in kernels) + " |")
    lines += ["", "Derived:", ""]
    for j, k in enumerate(kernels):
        m = mean[k]
        d = sum(durs[k]) / len(durs[k]) / 1e3
        parts = [f"- kernel {j} ({d:.1f} us per profiled launch):"]
        if m.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs: an eighth of it is the launch's
            # length in shader-clock cycles, which over the launch's duration is the clock
            # (for launches of a few tens of microseconds the count also covers the
            # dispatch's set-up under counter collection, so the clock is given for
            # long launches only and the busy share below is a lower bound)
            gpu_cycles = m["GRBM_GUI_ACTIVE"] / 8
            parts.append(f"{gpu_cycles:.4g} GPU-active cycles" +
                         (f", i.e. a mean shader clock of {gpu_cycles / d / 1e3:.2f} GHz;" if d >= 100 else ";"))
        if m.get("SQ_INSTS_MFMA"):
            parts.append(f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / m['SQ_INSTS_MFMA']:.1f} matrix-core cycles "
                         f"per MFMA instruction, {m['SQ_INSTS_MFMA']:.4g} MFMA instructions;")
            if m.get("GRBM_GUI_ACTIVE"):
                # SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of all 1024 SIMDs (256 CUs x 4)
                parts.append(f"matrix cores busy {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / gpu_cycles:.1f}% "
                             f"of the launch's cycles;")
        if m.get("SQ_LDS_IDX_ACTIVE"):
            parts.append(f"LDS bank conflicts {100 * m.get('SQ_LDS_BANK_CONFLICT', 0) / m['SQ_LDS_IDX_ACTIVE']:.2f}% "
                         f"of LDS-active cycles;")
        if m.get("TCC_HIT_sum") is not None and m.get("TCC_MISS_sum"):
            parts.append(f"L2 hit rate {100 * m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.1f}%;")
        if m.get("SQ_INSTS_MFMA") and m.get("SQ_INSTS_VALU") is not None:
            parts.append(f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f} VALU instructions (MFMA included) "
                         f"per MFMA.")
        if m.get("TA_BUSY_avr") is not None and m.get("GRBM_GUI_ACTIVE"):
            # TA_TA_BUSY counts busy cycles per texture-addresser instance (one per CU);
            # a direct-to-LDS load is one TA_FLAT_READ_LDS wavefront of 1 KB
            gpu_cycles = m["GRBM_GUI_ACTIVE"] / 8
            parts.append(f"texture addressers busy {100 * m['TA_BUSY_avr'] / gpu_cycles:.1f}% of the launch's "
                         f"cycles on average ({100 * m.get('TA_BUSY_max', 0) / gpu_cycles:.1f}% at most);")
            if m.get("TA_FLAT_READ_LDS_WAVEFRONTS_sum"):
                lds_bytes = m["TA_FLAT_READ_LDS_WAVEFRONTS_sum"] * 1024
                parts.append(f"{lds_bytes / 2**20:.1f} MiB loaded straight into LDS, "
                             f"{lds_bytes / 256 / gpu_cycles:.1f} bytes per CU per cycle;")
        if m.get("SQ_WAVE_CYCLES") and m.get("SQ_WAIT_INST_ANY") is not None:
            parts.append(f"waves waiting on an instruction {100 * m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.0f}% "
                         f"of wave cycles.")
        lines.append(" ".join(parts))
    fname = ("counters_sgemm4096x4096x1024_hgemm4096cube.md" if name == "step" else f"counters_{_slug(name)}.md")
    path = os.path.join(ROOT, "profiles", fname)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)
    return 0


def write_resources() -> int:
    """The compiler's resource usage (hipcc kernel-resource-usage remarks) of the kernels
    that the committed counter summaries profile, and a summary over every kernel
    instantiation, as profiles/resources.md."""
    import glob

    from dense_gemm_optimisation_f32_amd import build

    recs = build.resource_usage()
    by_name = {_short(r["kernel"]): r for r in recs}
    # the kernels of each profiled configuration, as the counter summaries name them
    used = {}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "counters_*.md"))):
        cfg = os.path.basename(path)[len("counters_"):-3]
        for line in open(path):
            m = re.match(r"- kernel \d+: `(.+)`$", line.strip())
            if m:
                used.setdefault(m.group(1).split("<mi355gemm::")[0], []).append(cfg)
    lds_cu = 160 * 1024

    def row(name, cfgs):
        r = by_name.get(name)
        if r is None:
            return f"| `{name}` | {', '.join(cfgs)} | not found in the sources | | | | | | |"
        lds = int(r.get("LDS Size [bytes/block]", 0))
        wg_cu = lds_cu // lds if lds else "-"
        return (f"| `{name}` | {', '.join(cfgs)} | {r['VGPRs']} | {r['AGPRs']} | {r['TotalSGPRs']} | "
                f"{r['ScratchSize [bytes/lane]']} | {r['VGPRs Spill']} / {r['SGPRs Spill']} | "
                f"{lds // 1024} KiB ({wg_cu}) | {r['Occupancy [waves/SIMD]']} |")

    lines = ["# Compiler resource usage of the profiled kernels", "",
             "Command (hipcc's kernel-resource-usage remarks on the committed sources; no GPU):", "",
             "```", "python3 $R/bench.py --write-resources   # R = repository root", "```", "",
             "Per kernel: architectural VGPRs and accumulation VGPRs (AGPRs) per lane, SGPRs, scratch "
             "bytes per lane, spilled VGPRs / SGPRs, LDS per work-group (in brackets the work-groups "
             "that fit in a CU's 160 KiB), and the waves per SIMD the registers allow (the compiler's "
             "occupancy figure). The configurations are those of profiles/counters_*.md that launch the "
             "kernel.", "",
             "| kernel | profiled in | VGPRs | AGPRs | SGPRs | scratch (B/lane) | spills V / S | LDS per WG | "
             "waves per SIMD |", "|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(used):
        lines.append(row(name, sorted(set(used[name]))))
    lines += ["", "Every kernel instantiation in the sources:", "",
              "| source | kernels | max VGPRs | max AGPRs | with scratch | with VGPR spills | with SGPR spills |",
              "|---|---|---|---|---|---|---|"]
    for src in sorted({r["source"] for r in recs}):
        rs = [r for r in recs if r["source"] == src]
        lines.append(f"| {src} | {len(rs)} | {max(int(r['VGPRs']) for r in rs)} | "
                     f"{max(int(r['AGPRs']) for r in rs)} | "
                     f"{sum(int(r['ScratchSize [bytes/lane]']) > 0 for r in rs)} | "
                     f"{sum(int(r['VGPRs Spill']) > 0 for r in rs)} | {sum(int(r['SGPRs Spill']) > 0 for r in rs)} |")
    spilled = [r for r in recs if int(r["VGPRs Spill"]) > 0 or int(r["SGPRs Spill"]) > 0
               or int(r["ScratchSize [bytes/lane]"]) > 0]
    if spilled:
        lines += ["", "Kernels with spills or scratch:", ""]
        for r in spilled:
            lines.append(f"- `{_short(r['kernel'])}`: VGPR spills {r['VGPRs Spill']}, SGPR spills "
                         f"{r['SGPRs Spill']}, scratch {r['ScratchSize [bytes/lane]']} B/lane")
    path = os.path.join(ROOT, "profiles", "resources.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)
    return 0


def write_traffic(name: str, fetch_csv: str, write_csv: str) -> int:
    """Per-launch HBM traffic of the library's kernels in a --profile NAME --copy-calibration
    run, from FETCH_SIZE / WRITE_SIZE counter runs, each scaled by the ratio of known
    bytes to counted bytes for the calibration copy.  The records are merged into the
    JSON block of profiles/hbm_traffic.md (step kernels under "sgemm" and "hgemm",
    other configurations under their names)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            kname, value = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0
            key = ("sgemm" if "sgemm" in kname else "hgemm") if "gemm" in kname else "copy"
            if key == "copy" and value < COPY_BYTES / 8:
                continue   # other small kernels of the run (tensor fills), not the calibration copy
            vals.setdefault(key, {}).setdefault(kname, []).append(value)
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def mean(d, key):
        items = d[key]
        allv = [x for v in items.values() for x in v]
        return " + ".join(sorted(items)), sum(allv) / len(allv)

    copy_name, copy_f = mean(fetch, "copy")
    _, copy_w = mean(write, "copy")
    scale_f, scale_w = COPY_BYTES / copy_f, COPY_BYTES / copy_w
    try:
        recs = _traffic_records()
    except (OSError, ValueError):
        recs = {}
    recs["copy_calibration"] = {"kernel": copy_name, "bytes": COPY_BYTES, "fetch_counted": copy_f,
                                "write_counted": copy_w, "fetch_scale": scale_f, "write_scale": scale_w}
    if name == "step":
        targets = [("sgemm", "sgemm", STEP_WORKLOADS["sgemm"],
                    4 * (4096 * 1024 * 2 + 4096 * 4096), "step"),
                   ("hgemm", "hgemm", STEP_WORKLOADS["hgemm"], 2 * (4096 * 4096 * 2) + 4 * 4096 * 4096, "step")]
    else:
        c = {x["name"]: x for x in extra_configs()}[name]
        kind = "sgemm" if c["kind"] == "f32" else "hgemm"
        targets = [(name, kind, name, config_bytes(c), name)]
        # the step's two calls are these configurations alone (same kernel, shape and data)
        step_of = {"sgemm_4096x4096x1024": "sgemm", "hgemm_4096^3": "hgemm"}
        if name in step_of:
            targets.append((step_of[name], kind, STEP_WORKLOADS[kind], config_bytes(c), name))
    for key, kind, workload, alg, prof in targets:
        kname, f = mean(fetch, kind)
        _, w = mean(write, kind)
        total = f * scale_f + w * scale_w
        recs[key] = {"kernel": kname, "workload": workload, "profile": prof, "source_sha": source_digest(kind),
                     "fetch_bytes_per_launch": f * scale_f, "write_bytes_per_launch": w * scale_w,
                     "hbm_bytes_per_launch": total, "algorithmic_bytes": alg}
    rows = []
    for key, r in recs.items():
        if key == "copy_calibration":
            continue
        rows.append(f"| {key} | {r['workload']} | {r['fetch_bytes_per_launch'] / 1e6:.1f} | "
                    f"{r['write_bytes_per_launch'] / 1e6:.1f} | {r['hbm_bytes_per_launch'] / 1e6:.1f} | "
                    f"{r['algorithmic_bytes'] / 1e6:.1f} | {r['hbm_bytes_per_launch'] / r['algorithmic_bytes']:.2f} |")
    cmd = ("cd /tmp && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/traffic_fetch -o t -- "
           "python3 $R/bench.py --profile NAME --steps 3 --warmup 1 --copy-calibration\n"
           "cd /tmp && timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/traffic_write -o t -- "
           "python3 $R/bench.py --profile NAME --steps 3 --warmup 1 --copy-calibration\n"
           "python3 $R/bench.py --write-traffic NAME $OUT/traffic_fetch/t_counter_collection.csv "
           "$OUT/traffic_write/t_counter_collection.csv\n"
           "# R = repository root, OUT = an output directory, NAME = step or a configuration name")
    cal = recs["copy_calibration"]
    text = ("# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n"
            f"Commands (one MI355X):\n\n```\n{cmd}\n```\n\n"
            f"Calibration (latest run): a plain elementwise copy of {COPY_BYTES >> 20} MiB reads and writes "
            f"{COPY_BYTES} bytes; the counters read {cal['fetch_counted']:.0f} B fetched and "
            f"{cal['write_counted']:.0f} B written, so fetch counts are scaled by {cal['fetch_scale']:.4f} and "
            f"write counts by {cal['write_scale']:.4f}.\n\n"
            "| record | workload | fetched (MB) | written (MB) | total (MB) | algorithmic (MB) | ratio |\n"
            "|---|---|---|---|---|---|---|\n" + "\n".join(rows) + "\n\n"
            "Machine-readable copy (bench.py reads it; a record whose source_sha no longer matches the kernel "
            "source is ignored):\n\n```json\n" + json.dumps(recs, indent=1) + "\n```\n")
    with open(TRAFFIC_FILE, "w") as f:
        f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
