#!/usr/bin/env python3
"""Benchmark of the row-major FP32 GEMM C[M,K] = A[M,N] x B[N,K] on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]

One step is one call of the library's solve() on the workload's inputs,
which are already resident in HBM when the timed region starts. W untimed
steps, then exactly K steps between two device synchronisations on the host
clock. Without --warmup, W is as many steps as take about 0.3 s (at least 5):
the GPU's clock climbs over the first tens of milliseconds of work, which a
few launches of a small shape never reach. Prints ONE JSON line:

  value        whole-job throughput over the K steps (TFLOP/s = 2MNK / time;
               GB/s of algorithmic bytes for the matrix-vector workload)
  roofline     the kernel's average launch duration (the HIP event time
               around the K timed steps, one event pair on the stream they
               run on, over K; launch_ms adds the spread of single calls, each
               between its own event pair, from an untimed pass), its
               algorithmic FLOP (or bytes) per launch over that duration,
               against the MI355X peak; `traffic` = HBM bytes per launch from rocprofv3
               FETCH_SIZE / WRITE_SIZE counters (profiles/), or null if the
               kernel sources changed since those counters were taken;
               `counters` = the dominant kernel's matrix-core busy fraction,
               LDS busy fraction, LDS bank conflicts per access and MFMA
               FLOP / 2MNK from a rocprofv3 --pmc run (same file, same rule)
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload
               (leading rows of A, or the whole product repeated), on this
               host's cores
  batched      the same launches back to back between two events only
               (and, for calls under 0.2 ms, captured in one HIP graph and
               replayed, which takes the host's launch cost out)
  clock        cycles per launch (profiles/<workload>_clock.md, GPU-active
               clocks from rocprofv3) over this run's launch time: the clock
               the timed launches ran at, the FP32 matrix peak at that clock,
               and the cycle efficiency 2MNK / (256 FLOP x 256 CUs x cycles)
  read_ceiling (matrix-vector workload) the measured streaming-read rate of
               a plain 1 GiB read (fgr_stream_read), and the kernel's
               fraction of it
  parity       the timed run's C against the oracle product that the
               cpu_baseline leg computed (every element of the rows it
               covers: all of them when it ran the whole product): the
               largest |C - C_oracle| / (1e-5 S + 1e-6) and pass / fail

Workloads (seeded synthetic inputs, synth/): leetgpu8192 (default, the
LeetGPU timed shape M=8192, N=6144, K=4096, normal entries / sqrt(N)),
cube4096, ragged1023, cube256, gemv8192, longn128 (128 x 262144 x 128: few
output tiles, long reduction). For shapes whose reduction is split across
workgroups one step is two kernels (partial tiles, then their sum); the
roofline's launch duration covers both.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X: 256 CU x 256 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
WARMUP_SECONDS = 0.3  # default warm-up: the clock climbs over the first tens of ms of work
METRIC = "FP32 GEMM TFLOP/s at M=8192,N=6144,K=4096; % of MI355X FP32 MFMA peak"
# every source the library is built from (csrc/*.hpp and csrc/*.hip)
KERNEL_SOURCES = sorted(n for n in os.listdir(os.path.join(ROOT, "fp32_gemm_row_amd", "csrc"))
                        if n.endswith((".hpp", ".hip")))
COPY_BYTES = 512 << 20


_CXX_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_text(source: str) -> str:
    """C++/HIP source with its comments removed and each run of blank space
    made one space: what the compiler sees, so that a profile stays current
    through edits of comments and layout alone."""
    text = _CXX_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), source)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """First 16 hex digits of the sha256 of the library's sources (csrc/*.hip,
    *.hpp, in name order) as code_text gives them. Profile summaries record it;
    their counters are used only while it still matches."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp32_gemm_row_amd", "csrc", name), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
            h.update(b"\0")
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch from profiles/<workload>_traffic.md, if current."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    src = re.search(r"kernel-source-sha256:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm-bytes-per-launch:\s*([0-9]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return int(val.group(1))


CU_COUNT = 256
FP32_FLOP_PER_CU_CLK = 256  # v_mfma_f32_32x32x2_f32: 4096 FLOP in 64 cycles, 4 SIMDs per CU
NUM_XCC = 8


def recorded_clock(workload: str):
    """The dominant kernel's GPU-active cycles per launch from
    profiles/<workload>_clock.md, if current (same kernel sources)."""
    rec = recorded_cycles(workload)
    return rec[0] if rec else None


def recorded_cycles(workload: str):
    """(GPU-active cycles, shader-engine busy cycles or None) per launch from
    profiles/<workload>_clock.md, if current (same kernel sources)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_clock.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    src = re.search(r"kernel-source-sha256:\s*([0-9a-f]+)", text)
    cyc = re.search(r"^cycles-per-launch:\s*([0-9.]+)", text, flags=re.M)
    busy = re.search(r"^busy-cycles-per-launch:\s*([0-9.]+)", text, flags=re.M)
    if not src or not cyc or src.group(1) != kernel_source_hash():
        return None
    return float(cyc.group(1)), float(busy.group(1)) if busy else None


def summarize_clock(workload, pmc_dir, commands, out_path, warmup=2):
    """profiles/<workload>_clock.md from a rocprofv3 --pmc GRBM_GUI_ACTIVE
    SQ_BUSY_CYCLES SQ_CYCLES --kernel-trace run: per dispatch of the dominant
    kernel, GPU-active cycles (GRBM_GUI_ACTIVE summed over the XCDs, divided
    by their number), the dispatch's duration and the clock they imply; the
    kernel's cycles per launch set against the cycles its 2MNK FLOP take at
    the matrix cores' rate (256 FLOP per CU per clock), a clock-independent
    efficiency."""
    rows = _csv_rows(_find(pmc_dir, "counter_collection.csv"))
    trace = {r["Dispatch_Id"]: r for r in _csv_rows(_find(pmc_dir, "kernel_trace.csv"))}
    per = {}
    for r in rows:
        if "copyBuffer" in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {"kernel": r["Kernel_Name"]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    names = {}
    for d in per.values():
        names[d["kernel"]] = names.get(d["kernel"], 0) + d.get("GRBM_GUI_ACTIVE", 0)
    top = max(names, key=names.get)
    disp = sorted((int(k), v) for k, v in per.items() if v["kernel"] == top)[warmup:]
    import synth

    w = synth.WORKLOADS[workload]
    ideal = w.flops / (CU_COUNT * FP32_FLOP_PER_CU_CLK)
    lines = [
        f"# Clock and cycles: {top.split('(')[0]} on {workload} (M={w.M}, N={w.N}, K={w.K})",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; repository at /root/repo):",
        "",
        *[f"    {c}" for c in commands],
        "",
        f"GRBM_GUI_ACTIVE counts GPU-active clocks; rocprofv3 sums it over the {NUM_XCC} XCDs, so cycles = "
        f"GRBM_GUI_ACTIVE / {NUM_XCC}. SQ_CYCLES (summed over the 32 shader engines) and SQ_BUSY_CYCLES are shown "
        "beside it. Clock = cycles / dispatch duration (kernel trace of the same run; the profiler serialises "
        "dispatches, so the clock here ramps over the first ones). Ideal cycles = 2MNK / (256 CUs x 256 FLOP "
        f"per clock) = {ideal:.0f}. GRBM_GUI_ACTIVE can also count clocks outside a dispatch's trace window: "
        "for dispatches of tens of microseconds the clock column then reads above the chip's 2.4 GHz, and "
        "rocprofv3's MfmaUtil, whose denominator it is, reads low. The shader engines' busy cycles "
        "(SQ_BUSY_CYCLES / 32, the clocks in which an engine had waves) hold the kernel's own span; "
        "busy-cycle-efficiency sets the ideal cycles against them.",
        "",
        "| dispatch | duration ns | GRBM_GUI_ACTIVE / 8 | SQ_CYCLES / 32 | SQ_BUSY_CYCLES / 32 | clock GHz |",
        "|---|---|---|---|---|---|",
    ]
    cycles, busy = [], []
    for did, d in disp:
        t = trace.get(str(did))
        ns = int(t["End_Timestamp"]) - int(t["Start_Timestamp"]) if t else 0
        cyc = d.get("GRBM_GUI_ACTIVE", 0) / NUM_XCC
        cycles.append(cyc)
        busy.append(d.get("SQ_BUSY_CYCLES", 0) / 32)
        lines.append(f"| {did} | {ns} | {cyc:.0f} | {d.get('SQ_CYCLES', 0) / 32:.0f} | "
                     f"{d.get('SQ_BUSY_CYCLES', 0) / 32:.0f} | {cyc / ns if ns else 0:.3f} |")
    avg = sum(cycles) / len(cycles)
    avg_busy = sum(busy) / len(busy)
    lines += [
        "",
        f"cycles-per-launch: {avg:.0f}",
        f"busy-cycles-per-launch: {avg_busy:.0f}",
        f"ideal-mfma-cycles: {ideal:.0f}",
        f"cycle-efficiency: {ideal / avg:.4f}",
        f"busy-cycle-efficiency: {ideal / avg_busy:.4f}" if avg_busy else "busy-cycle-efficiency: n/a",
        "",
        f"kernel-source-sha256: {kernel_source_hash()}",
        "",
    ]
    with open(out_path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    return out_path


def summarize_read(trace_dir, commands, out_path, warmup=5):
    """profiles/stream_read_1gib.md from a rocprofv3 --kernel-trace --stats run
    of bench.py --read-ceiling: each grid size's launches (in launch order,
    warm-ups dropped) and their read rate over the 1 GiB buffer."""
    trace = [r for r in _csv_rows(_find(trace_dir, "kernel_trace.csv")) if "stream_read" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    groups = {}
    for r in trace:
        blocks = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0) // 256
        groups.setdefault(blocks, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = [
        "# Streaming-read ceiling: fgr_stream_read over 1 GiB (each float read once, 128-bit loads)",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; repository at /root/repo):",
        "",
        *[f"    {c}" for c in commands],
        "",
        "| workgroups | timed launches | average ns | min ns | GB/s at the average |",
        "|---|---|---|---|---|",
    ]
    best = 0.0
    for blocks, d in sorted(groups.items()):
        t = d[warmup:] or d
        avg = sum(t) / len(t)
        gbs = READ_BYTES / avg
        best = max(best, gbs)
        lines.append(f"| {blocks} | {len(t)} | {avg:.0f} | {min(t)} | {gbs:.1f} |")
    lines += ["", f"read-ceiling-gbs: {best:.1f}", "", f"kernel-source-sha256: {kernel_source_hash()}", ""]
    with open(out_path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    return out_path


def recorded_counters(workload: str):
    """Matrix-core and LDS counters of the dominant kernel from
    profiles/<workload>_traffic.md, if current (same kernel sources)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    src = re.search(r"kernel-source-sha256:\s*([0-9a-f]+)", text)
    if not src or src.group(1) != kernel_source_hash():
        return None
    out = {}
    for key in ("mfma-busy", "lds-bank-conflicts-per-access", "lds-busy", "mfma-flop-per-2mnk"):
        m = re.search(rf"{key}:\s*([0-9.eE+-]+)", text)
        if m:
            out[key.replace("-", "_")] = float(m.group(1))
    return out or None


def _csv_rows(path):
    import csv

    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _find(directory, suffix):
    for root, _, files in os.walk(directory):
        for name in files:
            if name.endswith(suffix):
                return os.path.join(root, name)
    raise FileNotFoundError(f"no *{suffix} under {directory}")


SQ_COUNTERS = ("MfmaUtil", "LdsUtil", "LdsBankConflict", "SQ_INSTS_VALU_MFMA_MOPS_F32")
CLOCK_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_CYCLES")
ABLATION_COUNTERS = ("MfmaUtil", "LdsUtil", "LdsBankConflict")


def profile_commands(kind, workload=None, warmup=5, out="/tmp/prof", summary_out=None):
    """The recipe behind a summary, written into it when no --command is given:
    the runs that fill the folders the summary reads (from /tmp with
    TMPDIR=/tmp, each under its own time limit) and the summarising call (from
    the repository root). Each --pmc pass is a run of its own."""
    b = "python3 /root/repo/bench.py"
    fmt = "--output-format csv --"
    if kind == "traffic":
        w, d = f"--workload {workload} --no-cpu-baseline", f"{out}/{workload}"
        return [
            f"rocprofv3 --kernel-trace --stats -d {d}/kt -o kt {fmt} {b} {w} --steps 20 --warmup {warmup}",
            f"rocprofv3 --pmc FETCH_SIZE -d {d}/pmc_fetch -o pmc {fmt} {b} {w} --steps 3 --warmup 1 --calibrate-copy",
            f"rocprofv3 --pmc WRITE_SIZE -d {d}/pmc_write -o pmc {fmt} {b} {w} --steps 3 --warmup 1 --calibrate-copy",
            f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} -d {d}/pmc_sq -o pmc {fmt} {b} {w} --steps 3 --warmup 1",
            f"python3 bench.py --workload {workload} --warmup {warmup} --summarize {d}/kt {d}/pmc_fetch "
            f"{d}/pmc_write --summarize-sq {d}/pmc_sq",
        ]
    if kind == "clock":
        return [
            f"rocprofv3 --pmc {' '.join(CLOCK_COUNTERS)} --kernel-trace -d {out}/clk -o clk {fmt} {b} "
            f"--workload {workload} --no-cpu-baseline --steps 10 --warmup 2",
            f"python3 bench.py --workload {workload} --summarize-clock {out}/clk"
            + (f" --summary-out {summary_out}" if summary_out else ""),
        ]
    if kind == "read":
        return [
            f"rocprofv3 --kernel-trace --stats -d {out}/rd -o rd {fmt} {b} --read-ceiling --steps 20 --warmup {warmup}",
            f"python3 bench.py --summarize-read {out}/rd",
        ]
    if kind == "ablation":
        return [
            f"{b} --workload {workload} --ablation --steps 20 --warmup 5 > {out}/ablation.jsonl",
            f"rocprofv3 --pmc {' '.join(ABLATION_COUNTERS)} -d {out}/abl_sq -o pmc {fmt} {b} --workload {workload} "
            "--ablation --steps 3 --warmup 1",
            "python3 -m fp32_gemm_row_amd.build --resource-report profiles/kernel_resources.md",
            f"python3 bench.py --workload {workload} --summarize-ablation {out}/ablation.jsonl {out}/abl_sq "
            "profiles/kernel_resources.md",
        ]
    raise ValueError(kind)


def summarize_profiles(workload, trace_dir, fetch_dir, write_dir, commands, out_path, warmup=5, sq_dir=None):
    """Write the rocprofv3 summary of one workload's dominant kernel.

    trace_dir: a --kernel-trace --stats run; fetch_dir / write_dir: --pmc
    FETCH_SIZE / WRITE_SIZE runs of bench.py --calibrate-copy. Each counter
    is scaled by (known bytes of the plain 512 MiB device copy) / (what the
    same counter reads for that copy). sq_dir (optional): a --pmc run of
    rocprofv3's derived MfmaUtil (matrix-core busy cycles over GPU-active
    cycles times SIMDs, percent), LdsUtil (percent), LdsBankConflict (bank
    conflict cycles per conflict-free LDS cycle) and the raw
    SQ_INSTS_VALU_MFMA_MOPS_F32 (FP32 MFMA multiply-or-add operations / 512)."""
    stats = _csv_rows(_find(trace_dir, "kernel_stats.csv"))
    stats.sort(key=lambda r: float(r["TotalDurationNs"]), reverse=True)
    # the product's kernels only: not the read-ceiling measurement or torch's own
    top = [r for r in stats if "fgr::" in r["Name"] and "stream_read" not in r["Name"]][0]
    # the dispatches of the timed steps: drop the warm-up launches
    trace = [r for r in _csv_rows(_find(trace_dir, "kernel_trace.csv")) if r["Kernel_Name"] == top["Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    timed = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace[warmup:]]
    timed_avg = sum(timed) / len(timed)

    def per_dispatch(directory, counter):
        rows = _csv_rows(_find(directory, "counter_collection.csv"))
        kern = [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and r["Kernel_Name"] == top["Name"]]
        # the 512 MiB calibration copies: the copy dispatches with the largest
        # grid (small device-to-host copies use the same kernel)
        copies = [r for r in rows if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
        big = max((int(r["Grid_Size"]) for r in copies), default=0)
        copy = [float(r["Counter_Value"]) for r in copies if int(r["Grid_Size"]) == big]
        if not kern or not copy:
            raise ValueError(f"{counter}: kernel or copy dispatches missing in {directory}")
        k_kib = sum(kern) / len(kern)
        c_kib = sum(copy) / len(copy)
        factor = COPY_BYTES / (c_kib * 1024.0)
        return k_kib, c_kib, factor

    f_k, f_c, f_fac = per_dispatch(fetch_dir, "FETCH_SIZE")
    w_k, w_c, w_fac = per_dispatch(write_dir, "WRITE_SIZE")
    fetch_bytes = f_k * 1024.0 * f_fac
    write_bytes = w_k * 1024.0 * w_fac
    total = int(round(fetch_bytes + write_bytes))

    import synth

    w = synth.WORKLOADS[workload]
    lines = [
        f"# rocprofv3 summary: {top['Name']} on {workload} (M={w.M}, N={w.N}, K={w.K})",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; repository at /root/repo):",
        "",
        *[f"    {c}" for c in commands],
        "",
        "## Kernel trace (--kernel-trace --stats)",
        "",
        "| kernel | calls | average ns | min ns | max ns |",
        "|---|---|---|---|---|",
        *[f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |" for r in stats],
        "",
        f"Timed dispatches (the {len(timed)} after the {warmup} warm-up launches): average "
        f"{timed_avg:.0f} ns, min {min(timed)} ns, max {max(timed)} ns.",
        "",
        f"FLOP per launch 2MNK = {w.flops}: {w.flops / timed_avg / 1e3:.2f} TFLOP/s at the timed average. "
        f"Algorithmic bytes 4(MN+NK+MK) = {w.algorithmic_bytes}: {w.algorithmic_bytes / timed_avg:.1f} GB/s.",
        f"timed-average-ns: {timed_avg:.0f}",
        "",
        "## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE, KiB per dispatch)",
        "",
        "| counter | kernel KiB/dispatch | 512 MiB copy KiB/dispatch | scale (copy bytes / counter bytes) | kernel bytes |",
        "|---|---|---|---|---|",
        f"| FETCH_SIZE | {f_k:.1f} | {f_c:.1f} | {f_fac:.4f} | {fetch_bytes:.0f} |",
        f"| WRITE_SIZE | {w_k:.1f} | {w_c:.1f} | {w_fac:.4f} | {write_bytes:.0f} |",
        "",
        f"hbm-bytes-per-launch: {total}",
        f"ratio to algorithmic bytes: {total / w.algorithmic_bytes:.2f}",
        "",
    ]
    if sq_dir is not None:
        rows = _csv_rows(_find(sq_dir, "counter_collection.csv"))
        kernels = []
        for r in rows:
            if "copyBuffer" not in r["Kernel_Name"] and r["Kernel_Name"] not in kernels:
                kernels.append(r["Kernel_Name"])

        def avg(kernel, counter):
            v = [float(r["Counter_Value"]) for r in rows
                 if r["Kernel_Name"] == kernel and r["Counter_Name"] == counter]
            return (sum(v) / len(v), len(v)) if v else (float("nan"), 0)

        lines += [
            "## Matrix cores and LDS (--pmc " + " ".join(SQ_COUNTERS) + ", averages per dispatch)",
            "",
            "MFMA busy = MfmaUtil (percent of GPU-active cycles x SIMDs with the matrix unit busy); "
            "MFMA FLOP = 512 x SQ_INSTS_VALU_MFMA_MOPS_F32 (zero-padded edge tiles count too); "
            "LDS bank conflicts = conflict cycles per conflict-free LDS cycle.",
            "",
            "| kernel | dispatches | MFMA busy % | MFMA FLOP / dispatch | LDS busy % | LDS bank conflicts |",
            "|---|---|---|---|---|---|",
        ]
        for k in kernels:
            mu, n = avg(k, "MfmaUtil")
            lines.append(f"| {k} | {n} | {mu:.1f} | {avg(k, 'SQ_INSTS_VALU_MFMA_MOPS_F32')[0] * 512:.4g} "
                         f"| {avg(k, 'LdsUtil')[0]:.2f} | {avg(k, 'LdsBankConflict')[0]:.4f} |")
        mops = avg(top["Name"], "SQ_INSTS_VALU_MFMA_MOPS_F32")[0]
        lines += [
            "",
            f"Dominant kernel: mfma-busy: {avg(top['Name'], 'MfmaUtil')[0] / 100:.4f}",
            f"lds-busy: {avg(top['Name'], 'LdsUtil')[0] / 100:.4f}",
            f"lds-bank-conflicts-per-access: {avg(top['Name'], 'LdsBankConflict')[0]:.4f}",
            f"mfma-flop-per-2mnk: {mops * 512 / w.flops:.4f}",
            "",
        ]
    lines += [f"kernel-source-sha256: {kernel_source_hash()}", ""]
    with open(out_path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    return out_path


def variant_kernel(name: str) -> str:
    """The kernel (as the resource report and rocprofv3 name it) behind a
    controlled-comparison variant name."""
    parts = name.split()
    if parts[0] == "direct":
        ring = int(parts[1][len("ring"):])
        return f"fgr::gemm_mfma_dma_kernel<fgr::DmaConfig<{ring}, true, true, true> >"
    bufs = 1 if parts[1] == "single" else 2
    bm, bn = (int(x) for x in parts[2].split("x"))
    bk = int(parts[3][len("bk"):])
    wn = 4 if bn == 256 else 2
    return f"fgr::gemm_mfma_kernel<fgr::MfmaConfig<{bm}, {bn}, {bk}, 2, {wn}, 1, {bufs}>, true>"


def summarize_ablation(workload, jsonl, sq_dir, resources, commands, out_path):
    """profiles/<workload>_controlled_comparison.md: each variant's time
    (bench.py --ablation), the compiler's resource report for its kernel, and
    rocprofv3 counters (--pmc MfmaUtil LdsUtil LdsBankConflict) for it."""
    rows = [json.loads(line) for line in open(jsonl) if line.startswith("{") and '"variant"' in line]
    res = {}
    for line in open(resources, encoding="utf-8"):
        m = re.match(r"\| `void (.*?)` \| (.*) \|$", line.strip())
        if m:
            res[m.group(1)] = [c.strip() for c in m.group(2).split("|")]
    counters = _csv_rows(_find(sq_dir, "counter_collection.csv"))

    def avg(kernel, counter):
        v = [float(r["Counter_Value"]) for r in counters
             if r["Counter_Name"] == counter and r["Kernel_Name"].startswith("void " + kernel + "(")]
        return sum(v) / len(v) if v else float("nan")

    import synth

    w = synth.WORKLOADS[workload]
    lines = [
        f"# Controlled comparison on {workload} (M={w.M}, N={w.N}, K={w.K})",
        "",
        "One variable at a time: LDS buffering (register-staged kernel with one LDS buffer, or two with",
        "register prefetch; direct-copy kernel with an LDS ring of 3, 4 or 5 stages), output tile and",
        "reduction chunk. Time: mean of per-launch HIP events. Resources: hipcc",
        "-Rpass-analysis=kernel-resource-usage. Counters: rocprofv3 --pmc, averages per dispatch.",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; repository at /root/repo):",
        "",
        *[f"    {c}" for c in commands],
        "",
        "| variant | ms | TFLOP/s | VGPRs | AGPRs | waves/SIMD | LDS bytes | spills | MFMA busy % | LDS busy % | LDS bank conflicts |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for r in rows:
        k = variant_kernel(r["variant"])
        vg, ag, occ, lds, spill, _ = (res.get(k) or ["?"] * 6)[:6]
        lines.append(f"| {r['variant']} | {r['kernel_ms']:.3f} | {r['tflops']:.1f} | {vg} | {ag} | {occ} | {lds} | "
                     f"{spill} | {avg(k, 'MfmaUtil'):.1f} | {avg(k, 'LdsUtil'):.2f} | {avg(k, 'LdsBankConflict'):.4f} |")
    lines += ["", f"kernel-source-sha256: {kernel_source_hash()}", ""]
    with open(out_path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    return out_path


def kernel_ms(fn, steps, warmup, stream):
    """Mean of per-launch HIP-event durations on `stream`."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps


def ablation(w, dA, dBs, dC, copies, steps, warmup, stream):
    """Every (path, tile) the library accepts for this workload, then every
    controlled-comparison kernel variant (LDS buffering x output tile x
    reduction chunk), timed alike."""
    import fp32_gemm_row_amd as fgr

    variants = [(fgr.PATH_MFMA_DMA, 256), (fgr.PATH_MFMA_DMA_TAIL, 256)]
    for tile in (256, 128, 64):
        variants += [(fgr.PATH_MFMA_VEC, tile), (fgr.PATH_MFMA_SCALAR, tile)]
    for tile in (128, 64, 32, fgr.TILE_32X128):
        variants += [(fgr.PATH_MFMA_KSPLIT, tile), (fgr.PATH_MFMA_SPLITK, tile)]
    variants += [(fgr.PATH_MFMA_KSPLIT_TAIL, 128), (fgr.PATH_MFMA_KSPLIT_TAIL, 64),
                 (fgr.PATH_MFMA_SPLIT, 64), (fgr.PATH_MFMA_SPLIT, 32), (fgr.PATH_VALU, 128),
                 (fgr.PATH_GEMV_VEC, 0), (fgr.PATH_GEMV_SCALAR, 0)]
    auto = (fgr.select_path(dA, dBs[0], dC, w.M, w.N, w.K), fgr.select_tile(dA, dBs[0], dC, w.M, w.N, w.K))
    for path, tile in variants:
        def fn(i, path=path, tile=tile):
            fgr.solve_path(dA, dBs[i % copies], dC, w.M, w.N, w.K, path, tile, stream=stream)

        try:
            fn(0)
        except fgr.GemmError:
            continue  # this variant cannot run the shape
        ms = kernel_ms(fn, steps, warmup, stream)
        print(json.dumps({
            "workload": w.name, "path": fgr.PATH_NAMES[path], "tile": tile,
            "auto": (path, tile) == auto, "kernel_ms": round(ms, 5),
            "tflops": round(w.flops / ms / 1e9, 3), "gbs": round(w.algorithmic_bytes / ms / 1e6, 1),
        }), flush=True)
    # the controlled comparison: one kernel variant per buffering x tile x chunk
    for v, name in enumerate(fgr.variant_names()):
        def fn(i, v=v):
            fgr.solve_variant(dA, dBs[i % copies], dC, w.M, w.N, w.K, v, stream=stream)

        try:
            fn(0)
        except fgr.GemmError:
            continue
        ms = kernel_ms(fn, steps, warmup, stream)
        print(json.dumps({
            "workload": w.name, "variant": name, "kernel_ms": round(ms, 5),
            "tflops": round(w.flops / ms / 1e9, 3),
        }), flush=True)
    return 0


def roundtrip(w, A, B, dA, dB, dC, dev, iters=10):
    """Host round trip: pinned A, B -> device, solve, device C -> pinned host."""
    import torch

    import fp32_gemm_row_amd as fgr

    hA = torch.from_numpy(A.ravel()).pin_memory()
    hB = torch.from_numpy(B.ravel()).pin_memory()
    hC = torch.empty(w.M * w.K, dtype=torch.float32).pin_memory()

    def once():
        dA.copy_(hA, non_blocking=True)
        dB.copy_(hB, non_blocking=True)
        fgr.solve(dA, dB, dC, w.M, w.N, w.K)
        hC.copy_(dC, non_blocking=True)
        torch.cuda.synchronize()

    once()
    t0 = time.perf_counter()
    for _ in range(iters):
        once()
    ms = (time.perf_counter() - t0) / iters * 1e3
    return {
        "ms": round(ms, 4),
        "tflops": round(w.flops / ms / 1e9, 3),
        "pcie_bytes": w.algorithmic_bytes,
        "iterations": iters,
    }


def cpu_baseline(w, A, B, target_s: float, threads: int = 0):
    """Time the oracle on the first R rows of A (R sized for about target_s).

    Returns (record, (R, C, S)): the JSON record, and the oracle's fp64
    product and |a||b| sums of rows 0..R-1 from its first timed run (the whole
    product when R == M), which the parity check compares the GPU's output
    with. threads <= 0: every host thread."""
    import oracle

    threads = threads if threads > 0 else oracle.max_threads()
    rows = min(8, w.M)
    while True:  # probe until a timing is long enough to extrapolate from
        t0 = time.perf_counter()
        first = oracle.gemm(A[:rows], B, threads=threads)
        probe = time.perf_counter() - t0
        if probe >= 0.5 or rows >= w.M:
            break
        rows = min(w.M, rows * 4)
    R = max(rows, min(w.M, int(rows * target_s / max(probe, 1e-6))))
    elapsed = probe
    if R > rows:
        t0 = time.perf_counter()
        first = oracle.gemm(A[:R], B, threads=threads)
        elapsed = time.perf_counter() - t0
    # a whole product shorter than the target: repeat it
    reps = 1
    if R == w.M and elapsed < target_s / 2:
        reps = max(1, min(100000, int(target_s / max(elapsed, 1e-6))))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.gemm(A, B, threads=threads)
        elapsed = time.perf_counter() - t0
    flops = 2.0 * R * w.N * w.K * reps
    if w.M == 1:
        value = 4.0 * (R * w.N + w.N * w.K + R * w.K) * reps / elapsed / 1e9
        unit = "GB/s"
    else:
        value = flops / elapsed / 1e12
        unit = "TFLOP/s"
    what = f"rows 0..{R - 1} of A against all of B ({R}x{w.N}x{w.K}, fp64 with |a||b| sums)"
    if reps > 1:
        what = f"the whole product ({w.M}x{w.N}x{w.K}, fp64 with |a||b| sums) {reps} times"
    record = {
        "value": round(value, 6),
        "unit": unit,
        "cores": threads,
        "kind": "oracle",
        "sample": f"{what}, {elapsed:.2f} s",
    }
    return record, (R, first[0], first[1])


def parity_record(C, reference):
    """Every output of rows 0..R-1 of the GPU's C (numpy float32, M x K)
    against the oracle's product of those rows: finite, and |C - Cref| <=
    1e-5 S + 1e-6 element by element."""
    import numpy as np

    R, Cref, S = reference
    got = C[:R].astype(np.float64)
    finite = bool(np.isfinite(got).all())
    ratio = float(np.max(np.abs(got - Cref) / (1e-5 * S + 1e-6))) if finite else float("inf")
    return {
        "elements": int(got.size),
        "rows": int(R),
        "max_err_over_tol": round(ratio, 6),
        "finite": finite,
        "pass": finite and ratio <= 1.0,
        "bar": "|C - C_oracle| <= 1e-5 * sum_n |A[m,n]||B[n,k]| + 1e-6 per element (fp64 oracle)",
    }


def batched_ms(fn, launches, stream):
    """Mean time per launch of `launches` back-to-back launches between two HIP
    events on `stream` (no per-launch events: for kernels shorter than an
    event pair's own cost, as the tutorial's section 3 times its kernels)."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(launches):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / launches


def graph_ms(fn, launches, stream):
    """Mean time per launch of `launches` launches captured in one HIP graph,
    replayed between two events (after a first replay). The graph holds only
    the library's kernel launches (and, for split paths, its stream-ordered
    workspace allocation)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(launches):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / launches
    del graph
    return ms


READ_BYTES = 1 << 30  # the streaming-read buffer: 4x the 256 MB last-level cache


def read_ceiling(dev, stream, cus, steps=20, warmup=5):
    """The device's streaming-read rate: fgr_stream_read over a 1 GiB buffer
    (each float read once, 128-bit loads), per-launch HIP events, for a few
    grid sizes; the best one is the measured read ceiling."""
    import torch

    import fp32_gemm_row_amd as fgr

    n = READ_BYTES // 4
    X = torch.ones(n, dtype=torch.float32, device=dev)
    sweep = []
    for per_cu in (1, 2, 4, 8, 16):
        blocks = cus * per_cu
        out = torch.empty(blocks, dtype=torch.float32, device=dev)

        def fn(i, out=out, blocks=blocks):
            fgr.stream_read(X, n, out, blocks, stream=stream)

        ms = kernel_ms(fn, steps, warmup, stream)
        if not torch.isfinite(out).all():
            raise RuntimeError("stream_read produced non-finite sums")
        sweep.append({"blocks": blocks, "ms": round(ms, 5), "gbs": round(READ_BYTES / ms / 1e6, 1)})
    best = max(sweep, key=lambda r: r["gbs"])
    del X
    return {"bytes": READ_BYTES, "gbs": best["gbs"], "blocks": best["blocks"], "sweep": sweep}


TS_WORDS = 8  # 64-bit words per timestamp record (include/fp32_gemm_row_timestamps.h)


def timestamps_summary(w, path_name, tile, parts, launches_records, out_path, command):
    """profiles/<workload>_timestamps.md from the measurement build's
    per-workgroup records of several launches: the launch's span, the XCDs'
    staggered starts, each XCD's shader clock and loop cycles, and the loop
    cycles against the MFMA cycles the workgroup's work needs."""
    import numpy as np

    tile_rows = 32 if tile == 32128 else tile
    tile_cols = 128 if tile == 32128 else tile
    # MFMA cycles of one wave: a workgroup's tile over its part of N, its work
    # spread over 4 SIMDs at 64 FLOP per clock each (v_mfma_f32_32x32x2_f32)
    ideal = None
    if tile_rows and path_name.startswith("mfma_"):
        ideal = 2.0 * tile_rows * tile_cols * (w.N / max(1, parts)) / (4 * 64)
    per_launch = []
    xcd_rows = {}
    for rec in launches_records:
        r = rec[rec[:, 0] != 0]
        tiles = r[r[:, 6] == 0]
        if len(tiles) == 0:
            continue
        t0 = r[:, 0].min()
        span_us = (r[:, 2].max() - t0) / 100.0
        loop_us = (tiles[:, 1] - tiles[:, 0]) / 100.0
        end_us = (tiles[:, 2] - tiles[:, 1]) / 100.0
        cycles = (tiles[:, 4] - tiles[:, 3]).astype(np.float64)
        ghz = cycles / ((tiles[:, 1] - tiles[:, 0]) * 10.0)
        xcc = (tiles[:, 5] >> 32) & 0xFFFF
        starts = {}
        for x in sorted(set(xcc.tolist())):
            m = xcc == x
            starts[x] = (tiles[m, 0].min() - t0) / 100.0
            xcd_rows.setdefault(x, []).append((starts[x], float(np.median(ghz[m])), float(np.median(cycles[m])),
                                               float(np.median(loop_us[m]))))
        per_launch.append({
            "workgroups": len(r), "tiles": len(tiles), "span": span_us,
            "loop": float(np.median(loop_us)), "end": float(np.median(end_us)),
            "cycles": float(np.median(cycles)), "stagger": max(starts.values()) - min(starts.values()),
            "ghz_lo": float(min(np.median(ghz[xcc == x]) for x in starts)),
            "ghz_hi": float(max(np.median(ghz[xcc == x]) for x in starts)),
        })
    if not per_launch:
        raise RuntimeError("no timestamp records (does the plan's kernel record them?)")
    med = lambda k: float(np.median([d[k] for d in per_launch]))  # noqa: E731
    lines = [
        f"# Per-workgroup timestamps: {w.name} (M={w.M}, N={w.N}, K={w.K}), plan {path_name} {tile}"
        + (f", {parts} parts" if parts > 1 else ""),
        "",
        "Command (repository at /root/repo; the measurement build libfp32_gemm_row_ts.so, the same kernels",
        "with per-workgroup records of the constant 100 MHz clock and the shader clock):",
        "",
        f"    {command}",
        "",
        f"{len(per_launch)} launches, each after a synchronisation (so they start from an idle GPU), after",
        "0.3 s of warm-up launches. A workgroup's loop is its start to the end of its main loop; its end",
        "phase is the reduction of partial tiles (k-split kernels), the stores, and their completion.",
        "Medians over the launches (and over each launch's workgroups):",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| workgroups recorded per launch (tiles) | {per_launch[0]['workgroups']} ({per_launch[0]['tiles']}) |",
        f"| launch span, first start to last end | {med('span'):.2f} us |",
        f"| last XCD's first start after the first XCD's | {med('stagger'):.2f} us |",
        f"| a tile workgroup's loop | {med('loop'):.2f} us, {med('cycles'):.0f} shader clocks |",
        f"| a tile workgroup's end phase | {med('end'):.2f} us |",
        f"| shader clock, slowest to fastest XCD | {med('ghz_lo'):.3f} - {med('ghz_hi'):.3f} GHz |",
    ]
    if ideal:
        lines.append(f"| MFMA clocks of a wave's share of its tile (2 BM BN N_part / 256) | {ideal:.0f} "
                     f"(loop at {ideal / med('cycles') * 100:.1f}% of them) |")
    lines += ["", "Per XCD (medians over launches: first start after the launch's first, the XCD's tiles' clock,",
              "loop clocks and loop time):", "",
              "| XCD | first start, us | clock, GHz | loop clocks | loop, us |", "|---|---|---|---|---|"]
    for x in sorted(xcd_rows):
        v = np.array(xcd_rows[x])
        lines.append(f"| {x} | {np.median(v[:, 0]):.2f} | {np.median(v[:, 1]):.3f} | {np.median(v[:, 2]):.0f} | "
                     f"{np.median(v[:, 3]):.2f} |")
    lines += ["", f"loop-clocks: {med('cycles'):.0f}", f"launch-span-us: {med('span'):.2f}",
              f"xcd-start-stagger-us: {med('stagger'):.2f}", "",
              f"kernel-source-sha256: {kernel_source_hash()}", ""]
    with open(out_path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    return out_path


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: about 0.3 s of steps, at least 5; 5 for the "
                         "summaries, the ablation and the read ceiling)")
    ap.add_argument("--workload", default="leetgpu8192")
    ap.add_argument("--shape", type=int, nargs=3, metavar=("M", "N", "K"), default=None,
                    help="time this shape instead of a named workload (uniform [-1,1) inputs, --seed)")
    ap.add_argument("--seed", type=int, default=9, help="input seed for --shape")
    ap.add_argument("--path", type=int, default=0, help="force an FGR path (0 = auto)")
    ap.add_argument("--tile", type=int, default=0, help="force an MFMA output tile (0 = auto)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="cycle through this many copies of B (0 = 4 for the matrix-vector workload, "
                         "whose 256 MiB B would otherwise partly stay in the 256 MB last-level cache; 1 otherwise)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="target length of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, run a plain 512 MiB device copy three times "
                         "(the known-size reference for HBM byte counters)")
    ap.add_argument("--roundtrip", action="store_true",
                    help="also time the host round trip of the tutorial's section 3 (pinned host A and B "
                         "copied in, solve, C copied out; 1 warm-up, 10 timed on the host clock) and "
                         "add it as 'roundtrip' (never the headline value)")
    ap.add_argument("--ablation", action="store_true",
                    help="time every path/tile the library accepts for the workload, print one JSON line "
                         "per variant and exit (the controlled comparison of the LeetGPU write-up)")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/<workload>_traffic.md from three rocprofv3 output folders and exit")
    ap.add_argument("--summarize-clock", metavar="PMC_DIR", default=None,
                    help="write profiles/<workload>_clock.md from a rocprofv3 --pmc GRBM_GUI_ACTIVE "
                         "SQ_BUSY_CYCLES SQ_CYCLES --kernel-trace run and exit")
    ap.add_argument("--summarize-read", metavar="TRACE_DIR", default=None,
                    help="write profiles/stream_read_1gib.md from a rocprofv3 --kernel-trace --stats run of "
                         "bench.py --read-ceiling and exit")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the streaming-read ceiling (fgr_stream_read over 1 GiB) and print it")
    ap.add_argument("--summarize-sq", metavar="SQ_DIR", default=None,
                    help="(with --summarize) a rocprofv3 --pmc " + " ".join(SQ_COUNTERS) + " run to add")
    ap.add_argument("--summarize-ablation", nargs=3, metavar=("ABLATION_JSONL", "SQ_DIR", "RESOURCES_MD"),
                    help="write profiles/<workload>_controlled_comparison.md from a bench.py --ablation "
                         "output, a rocprofv3 --pmc MfmaUtil LdsUtil LdsBankConflict run of it and the "
                         "resource report, and exit")
    ap.add_argument("--timestamps", action="store_true",
                    help="with the measurement build (libfp32_gemm_row_ts.so), record per-workgroup timestamps "
                         "of --steps launches of the workload, write profiles/<workload>_timestamps.md and exit")
    ap.add_argument("--summary-out", metavar="PATH", default=None,
                    help="(with --summarize-clock) write the summary here instead of profiles/<workload>_clock.md, "
                         "the record bench.py reads the clock from (for kernels too short for that record)")
    ap.add_argument("--command", action="append", default=[],
                    help="(with a --summarize option) a command that produced the folders, recorded in the "
                         "summary in place of the standard recipe (profile_commands)")
    args = ap.parse_args()
    auto_warmup = args.warmup is None
    if auto_warmup:
        args.warmup = 5

    if args.summarize_ablation:
        out = os.path.join(ROOT, "profiles", f"{args.workload}_controlled_comparison.md")
        cmds = args.command or profile_commands("ablation", args.workload)
        print(summarize_ablation(args.workload, *args.summarize_ablation, cmds, out))
        return 0
    if args.summarize_read:
        out = os.path.join(ROOT, "profiles", "stream_read_1gib.md")
        cmds = args.command or profile_commands("read", warmup=args.warmup)
        print(summarize_read(args.summarize_read, cmds, out, args.warmup))
        return 0
    if args.summarize_clock:
        out = args.summary_out or os.path.join(ROOT, "profiles", f"{args.workload}_clock.md")
        cmds = args.command or profile_commands("clock", args.workload, summary_out=args.summary_out)
        print(summarize_clock(args.workload, args.summarize_clock, cmds, out))
        return 0
    if args.summarize:
        out = os.path.join(ROOT, "profiles", f"{args.workload}_traffic.md")
        cmds = args.command or profile_commands("traffic", args.workload, args.warmup)
        print(summarize_profiles(args.workload, *args.summarize, cmds, out, args.warmup,
                                 sq_dir=args.summarize_sq))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(
            "bench.py measures one GPU only: the library has no multi-GPU path "
            "(sharding output rows across GPUs is a design note, not built). Use --gpus 1.",
            file=sys.stderr,
        )
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    import fp32_gemm_row_amd as fgr
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (no CPU fallback)", file=sys.stderr)
        return 2
    if args.timestamps:
        from fp32_gemm_row_amd import build as fgr_build

        fgr.load_library(fgr_build.TS_LIB_PATH)
    else:
        fgr.load_library()
    if args.read_ceiling:
        dev = torch.device("cuda:0")
        res = read_ceiling(dev, torch.cuda.current_stream(), torch.cuda.get_device_properties(dev).multi_processor_count,
                           steps=args.steps, warmup=args.warmup)
        print(json.dumps({"metric": "streaming read GB/s (fgr_stream_read, 1 GiB)", **res}), flush=True)
        return 0

    if args.shape:
        M, N, K = args.shape
        w = synth.Workload(f"shape{M}x{N}x{K}", M, N, K, "uniform", args.seed)
    else:
        w = synth.WORKLOADS[args.workload]
    A, B = synth.workload_inputs(w)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A.ravel()).to(dev)
    copies = args.rotate or (4 if w.M == 1 else 1)
    dBs = [torch.from_numpy(B.ravel()).to(dev) for _ in range(copies)]
    dB = dBs[0]
    dC = torch.empty(w.M * w.K, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    auto_path = fgr.select_path(dA, dB, dC, w.M, w.N, w.K)
    auto_tile = fgr.select_tile(dA, dB, dC, w.M, w.N, w.K)
    path = args.path or auto_path
    tile = args.tile or (auto_tile if path == auto_path else 0)
    stream = torch.cuda.current_stream()

    def step(i):
        fgr.solve_path(dA, dBs[i % copies], dC, w.M, w.N, w.K, path, tile, stream=stream)

    def step_current(i):  # on torch's current stream (a graph capture's, when capturing)
        fgr.solve_path(dA, dBs[i % copies], dC, w.M, w.N, w.K, path, tile)

    if args.timestamps:
        import ctypes

        import numpy as np

        lib = fgr.load_library()
        lib.fgr_timestamps_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
        lib.fgr_timestamps_read.restype = ctypes.c_int
        t_warm = time.perf_counter()
        i = 0
        while time.perf_counter() - t_warm < WARMUP_SECONDS:
            for _ in range(5):
                step(i)
                i += 1
            torch.cuda.synchronize()
        records = []
        for i in range(args.steps):
            step(i)
            torch.cuda.synchronize()
            buf = np.zeros((4096, TS_WORDS), dtype=np.uint64)
            rc = lib.fgr_timestamps_read(buf.ctypes.data, 4096)
            if rc != 0:
                raise RuntimeError(f"fgr_timestamps_read: {fgr.status_string(rc)}")
            records.append(buf.astype(np.int64))
        parts = fgr.select_parts(dA, dB, dC, w.M, w.N, w.K) if (path, tile) == (auto_path, auto_tile) else 1
        out = os.path.join(ROOT, "profiles", f"{w.name}_timestamps.md")
        cmd = " ".join(["python3 /root/repo/bench.py"] + sys.argv[1:])
        print(timestamps_summary(w, fgr.PATH_NAMES[path], tile, parts, records, out, cmd))
        return 0

    if args.ablation:
        # the clock climbs over the first tens of ms of work: warm up on the
        # automatic plan first, so that the first variant is timed at the
        # sustained clock like the others
        t_warm = time.perf_counter()
        i = 0
        while time.perf_counter() - t_warm < WARMUP_SECONDS:
            for _ in range(5):
                step(i)
                i += 1
            torch.cuda.synchronize()
        return ablation(w, dA, dBs, dC, copies, args.steps, args.warmup, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if auto_warmup:  # until about 0.3 s of steps have run (the clock has climbed)
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < WARMUP_SECONDS:
            for _ in range(5):
                step(args.warmup)
                args.warmup += 1
            torch.cuda.synchronize()

    # The timed region: K steps back to back, one HIP event pair around them
    # on the launch stream (an event record between steps costs the GPU about
    # 4.5 us each, measured, which small shapes would pay on every step).
    region_start = torch.cuda.Event(enable_timing=True)
    region_end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    region_start.record(stream)
    for i in range(args.steps):
        step(i)
    region_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = region_start.elapsed_time(region_end) / args.steps / 1e3

    # untimed: one event pair per launch, for the spread of single calls
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    # the same launches back to back between two events only
    batch_launches = max(50, args.steps)
    batch_ms = batched_ms(step, batch_launches, stream)
    ms_per_step = wall / args.steps * 1e3
    gemv = w.M == 1
    if gemv:
        value = w.algorithmic_bytes * args.steps / wall / 1e9
        unit = "GB/s"
        achieved = w.algorithmic_bytes / avg_launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        metric = "FP32 GEMV-shaped GEMM GB/s at M=1,N=8192,K=8192; % of MI355X HBM peak"
    else:
        value = w.flops * args.steps / wall / 1e12
        unit = "TFLOP/s"
        achieved = w.flops / avg_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_FP32_PEAK_TFLOPS, "unit": "TFLOP/s"}
        metric = METRIC if w.name == "leetgpu8192" else f"FP32 GEMM TFLOP/s at M={w.M},N={w.N},K={w.K}"
    roof["frac"] = round(achieved / roof["peak"], 4)
    roof["traffic"] = recorded_traffic(w.name)
    roof["counters"] = recorded_counters(w.name)
    roof["batched"] = {
        "launches": batch_launches,
        "ms_per_launch": round(batch_ms, 5),
        "achieved": round(w.algorithmic_bytes / batch_ms / 1e6, 2) if gemv else round(w.flops / batch_ms / 1e9, 3),
    }
    if batch_ms < 0.2:
        # short calls: the same launches captured in one HIP graph and replayed
        # between two events, so that the host's launch cost drops out
        g_ms = graph_ms(step_current, batch_launches, stream)
        roof["batched"]["graph_ms_per_launch"] = round(g_ms, 5)
        roof["batched"]["graph_achieved"] = (round(w.algorithmic_bytes / g_ms / 1e6, 2) if gemv
                                             else round(w.flops / g_ms / 1e9, 3))
    rec = recorded_cycles(w.name)
    cycles, busy_cycles = rec if rec else (None, None)
    if cycles and not gemv:
        # cycles per launch (profiles/<workload>_clock.md) over this run's launch
        # time: the clock the timed launches ran at, and the peak at that clock
        ghz = cycles / (avg_launch_s * 1e9)
        peak_at_clock = CU_COUNT * FP32_FLOP_PER_CU_CLK * ghz / 1e3
        roof["clock"] = {
            "cycles_per_launch": round(cycles),
            "ghz": round(ghz, 3),
            "peak_at_clock": round(peak_at_clock, 1),
            "frac_at_clock": round(achieved / peak_at_clock, 4),
            "cycle_efficiency": round(w.flops / (CU_COUNT * FP32_FLOP_PER_CU_CLK) / cycles, 4),
        }
        if busy_cycles:
            # against the clocks in which the shader engines had waves
            roof["clock"]["busy_cycle_efficiency"] = round(w.flops / (CU_COUNT * FP32_FLOP_PER_CU_CLK) / busy_cycles, 4)
    if gemv:
        # the measured streaming-read ceiling beside the datasheet peak
        ceiling = read_ceiling(dev, stream, torch.cuda.get_device_properties(dev).multi_processor_count)
        ceiling["frac"] = round(achieved / ceiling["gbs"], 4)
        roof["read_ceiling"] = ceiling
    roof["launch_ms"] = {
        "mean": round(avg_launch_s * 1e3, 4),  # the timed region's event time / K
        "event_pair_mean": round(sum(launch_ms) / len(launch_ms), 4),
        "event_pair_min": round(min(launch_ms), 4),
        "event_pair_max": round(max(launch_ms), 4),
    }

    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "M": w.M,
            "N": w.N,
            "K": w.K,
            "values": {"normal": "N(0,1)/sqrt(N)", "uniform": "U[-1,1)", "integer": "{-4..4}"}.get(w.dist, w.dist),
            "seed": w.seed,
            "path": fgr.PATH_NAMES.get(path, str(path)),
            "tile": tile,
            "b_copies": copies,
        },
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.roundtrip:
        out["roundtrip"] = roundtrip(w, A, B, dA, dB, dC, dev)
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = COPY_BYTES
    if not args.no_cpu_baseline:
        # the oracle's product from the baseline's first timed run also checks
        # the timed run's output, element by element
        C_gpu = dC.cpu().numpy().reshape(w.M, w.K)
        out["cpu_baseline"], reference = cpu_baseline(w, A, B, args.cpu_seconds)
        out["parity"] = parity_record(C_gpu, reference)
        del reference
        if w.flops < 1e10:
            # small workloads: the oracle on one host thread as well
            single, _ = cpu_baseline(w, A, B, min(args.cpu_seconds, 10.0), threads=1)
            out["cpu_baseline"]["single_thread"] = single
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
