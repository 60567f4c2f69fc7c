#!/usr/bin/env python3
"""Benchmark: forward + backward banded Sinkhorn attention on one MI355X.

Workload (the long-context configuration): B=1, H=8, L=32768, d=128, band
W=256 (offsets [-128, 127]), T=100 stopped base steps, R=2 tail steps,
uniform marginals, Q, K, V ~ N(0,1)/sqrt(d) and dO ~ N(0,1) rounded to
bf16 (seeded synthetic data); fp32 accumulation, fp64 Sinkhorn state.

One step = sinkattn_forward + sinkattn_backward over the whole batch (every
row of the hot path), inputs resident in HBM.  Prints ONE JSON line with the
throughput, the roofline of the dominant kernel (the fused Sinkhorn step,
timed per launch with HIP events on its stream, against the MFMA/exp peak
with the work counted per half-step: 4 d flops and 2 exps per band entry
per Sinkhorn step), the same workload with the R = 4 tail, the other
workloads' step times, and the float64 oracle timed on the host's cores on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--R 2] [--no-cpu-baseline]

Profile summaries (rocprofv3 CSV output -> the text and JSON files kept under
profiles/):

    python bench.py --summarize DIR
      DIR/trace: rocprofv3 --kernel-trace --stats --output-format csv run
      DIR/fetch, DIR/write: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of
      "bench.py --copy-calibration" (a 256 MiB device copy calibrates both)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/s at L=32768 W=256 T=100 R=2; % of MFMA/exp roofline"
CONFIG = dict(B=1, H=8, L=32768, d=128, W=256, T=100, R=2, dtype="bf16")
# Published MI355X peaks (dense): bf16 MFMA 2.5 PFLOP/s, fp32 MFMA 157.3 TFLOP/s.
PEAK_MFMA = {"bf16": 2.5e15, "f32": 157.3e12}
# Transcendental (v_exp_f32) issue rate: 256 CUs x 2.4 GHz x 32 lanes/clk
# (half the 64-lane fp32 VALU rate per CU).
PEAK_EXP = 256 * 2.4e9 * 32
PEAK_HBM = 8.0e12  # bytes/s, published MI355X HBM3E bandwidth
PMC_FILE = os.path.join(ROOT, "profiles", "iter_kernel_long_context_pmc.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "iter_kernel_long_context.txt")
COPY_BYTES = 256 << 20  # calibration copy: bytes read and bytes written
KERNEL_SOURCES = [os.path.join(ROOT, "entropic_ot_banded_amd", "csrc", f)
                  for f in ("forward.hip", "common.hpp", "geom.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def band_entries(n: int, W: int) -> int:
    """|Omega| of one sequence of n real tokens (band clipped at the ends)."""
    h1, h2 = W // 2, (W + 1) // 2 - 1
    tot = 0
    for i in range(n):
        tot += min(n - 1, i + h2) - max(0, i - h1) + 1
    return tot


def band_entries_fast(n: int, W: int) -> int:
    h1, h2 = W // 2, (W + 1) // 2 - 1
    h1, h2 = min(h1, n - 1), min(h2, n - 1)
    full = n * (h1 + h2 + 1)
    return full - h1 * (h1 + 1) // 2 - h2 * (h2 + 1) // 2


def work_counts(B, H, L, d, W, T, R):
    """Algorithmic work of one forward + backward.

    Executed schedule (this library): a fused step evaluates the band score
    once per Sinkhorn step (row and column updates share it) -> (T+R) score
    contractions of 2d flops per band entry; output: score + P V (4d);
    backward: dV sweep (4d), 2R-1 vector sweeps (2d each), dQ and dK sweeps
    (score, dP and the product: 6d each).  Exps: one per entry per sweep.
    Half-step counting: one score per half-step, 2(T+R) 2d + 4d forward and
    (4R+10) d backward; 2(T+R) + 1 + 2R + 1 exps.
    """
    omega = B * H * band_entries_fast(L, W)
    ex_flops = omega * ((T + R) * 2 * d + 4 * d + 4 * d + (2 * R - 1) * 2 * d + 12 * d)
    ex_exps = omega * ((T + R) + 1 + 1 + (2 * R - 1) + 2)
    sv_flops = omega * (2 * (T + R) * 2 * d + 4 * d + (4 * R + 10) * d)
    sv_exps = omega * (2 * (T + R) + 1 + 2 * R + 1)
    return omega, ex_flops, ex_exps, sv_flops, sv_exps


def step_bytes_per_launch(B, H, L, d, esize, SB, TL, TR, tail=False):
    """Algorithmic HBM bytes of one fused-step launch: every Q and K row once,
    a and b, v^(t-2) read, u and v written (fp64), the column partials
    written and read back (fp32, one per column plus the window overlap of
    each segment), and the tail copies of u, v on the R tail steps."""
    tokens = B * H * L
    per_tok = 2 * d * esize + 4 + 4 + 8 + 8 + 8
    per_tok += 2 * 4 * (1.0 + 16.0 * (TL + TR) / (SB * 128))
    if tail:
        per_tok += 16
    return tokens * per_tok


def step_geometry(B, H, L, W):
    """Tile geometry the library picks for the fused step (host side of
    sinkattn_forward): tiles left/right of the diagonal tile, rows per
    segment in 128-row blocks."""
    h1 = min(W // 2, L - 1)
    h2 = min((W + 1) // 2 - 1, L - 1)
    TL, TR = (h1 + 15) // 16, (15 + h2) // 16
    NT = TL + TR + 1
    for inst in (3, 5, 9, 17):
        if NT <= inst:
            TR += inst - NT
            break
    nblk = (L + 127) // 128
    SB = min(max(-(-(B * H * nblk) // 256), 1), nblk)
    return SB, TL, TR


def load_pmc(launch_units=None):
    """HBM traffic per Sinkhorn step of the fused step kernel from committed
    rocprofv3 counters (per dispatch / steps per dispatch), scaled by a
    copy-kernel calibration; None if absent or taken on different kernel
    sources."""
    try:
        with open(PMC_FILE) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    if pmc.get("kernel_source_hash") != kernel_source_hash():
        return None
    fetch = pmc["fetch_kib_per_step"] * pmc["fetch_scale"]
    write = pmc["write_kib_per_step"] * pmc["write_scale"]
    return (fetch + write) * 1024.0


PROF_ARGS = ("--no-cpu-baseline --converge-tol 0 --certificate-rmax 0 --contraction-block 0 --no-peaks "
             "--r4-steps 0 --no-other-configs")
TRACE_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             "-d $OUT/trace -o run -- python3 $REPO/bench.py --steps 5 --warmup 20 "
             + PROF_ARGS)
SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU "
               "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS GRBM_GUI_ACTIVE")
SQ_FILE = os.path.join(ROOT, "profiles", "iter_kernel_long_context_sq.txt")
PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {ctr} --output-format csv "
           "-d $OUT/{sub} -o run -- python3 $REPO/bench.py --steps 2 --warmup 1 "
           + PROF_ARGS + " --copy-calibration")


HOW = "Commands ($REPO = repository root, $OUT = output directory of the profile runs):"
SUMMARIZE_CMD = "python3 $REPO/bench.py --summarize $OUT"
# The persistent step launch is cooperative; rocprofv3 then ends with a
# segmentation fault in its own teardown after the program has finished and
# its output files are written.  The profile runs accept that status only when
# the program printed its result line.
EXIT_NOTE = ("  (exit status 0, or 139 from the profiler's teardown after a cooperative launch "
             "once the program has printed its result line and the CSV files are complete)")
TCC_COUNTERS = "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_DRAM_sum"
TCC_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + TCC_COUNTERS + " --output-format csv "
           "-d $OUT/tcc -o run -- python3 $REPO/bench.py --steps 2 --warmup 1 " + PROF_ARGS)
LDS_STRIDES = (256, 272, 288, 304, 320)
LDS_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS "
           "--output-format csv -d $OUT/lds -o run -- python3 $REPO/bench.py --lds-probe > $OUT/lds_probe.json")
LDS_FILE = os.path.join(ROOT, "profiles", "lds_read_patterns.txt")
SWEEP_FILE = os.path.join(ROOT, "profiles", "sweep_kernels_long_context.txt")
L2_FILE = os.path.join(ROOT, "profiles", "l2_dram_long_context.txt")


def steps_per_dispatch(name):
    """Sinkhorn steps one dispatch of the fused step kernel covers: all T + R
    of a forward for the persistent instance (template flag true), else 1."""
    return CONFIG["T"] + CONFIG["R"] if ", true>" in name else 1


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize(d):
    """Write the profile summaries kept under profiles/ from rocprofv3 CSV
    output in d/trace (kernel trace + stats), d/fetch and d/write (PMC)."""
    import glob
    traces = glob.glob(os.path.join(d, "trace", "*kernel_stats.csv"))
    if not traces:  # an LDS probe run only
        summarize_lds(d)
        return
    stats = _csv_rows(traces[0])
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["Kernel statistics of the long-context workload (B=1, H=8, L=32768, d=128, W=256,",
             "T=100, R=2, bf16 inputs): 5 timed + 2 warm-up forward+backward steps.",
             "", HOW, "  " + TRACE_CMD, "  " + SUMMARIZE_CMD, EXIT_NOTE, "",
             f"{'calls':>6} {'avg_us':>10} {'total_ms':>10} {'pct':>6}  kernel"]
    for r in stats[:24]:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}  {r['Name'][:110]}")
    it = [r for r in stats if "iter_kernel" in r["Name"]]
    if it:
        spd = steps_per_dispatch(it[0]["Name"])
        lines += ["", f"fused step (iter_kernel): {int(it[0]['Calls'])} dispatches of {spd} step(s), average "
                  f"{float(it[0]['AverageNs']) / 1e3:.2f} us per dispatch = "
                  f"{float(it[0]['AverageNs']) / 1e3 / spd:.2f} us per step "
                  f"(min {float(it[0]['MinNs']) / 1e3 / spd:.2f}, max {float(it[0]['MaxNs']) / 1e3 / spd:.2f})"]
        # the timed dispatches (the last 5 of the main workload: warm-up first)
        tr = glob.glob(os.path.join(d, "trace", "*kernel_trace.csv"))
        if tr:
            disp = [r for r in _csv_rows(tr[0]) if "iter_kernel" in r["Kernel_Name"]]
            disp.sort(key=lambda r: int(r["Start_Timestamp"]))
            us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 / spd for r in disp[-5:]]
            if us:
                lines.append(f"timed dispatches (the last {len(us)}): " + ", ".join(f"{x:.2f}" for x in us)
                             + f" us per step, average {sum(us) / len(us):.2f}")
    logf = os.path.join(d, "trace.log")
    if os.path.exists(logf):
        for ln in open(logf):
            if ln.startswith("{"):
                lines += ["", "bench.py line of the profiled run:", ln.strip()]
    pmc = {"kernel_source_hash": kernel_source_hash()}
    for ctr, sub, key in (("FETCH_SIZE", "fetch", "fetch"), ("WRITE_SIZE", "write", "write")):
        files = glob.glob(os.path.join(d, sub, "*counter_collection.csv"))
        if not files:
            continue
        rows = [r for r in _csv_rows(files[0]) if r["Counter_Name"] == ctr]
        itr = [r for r in rows if "iter_kernel" in r["Kernel_Name"]]
        itv = [float(r["Counter_Value"]) / steps_per_dispatch(r["Kernel_Name"]) for r in itr]
        cp = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not itv or not cp:
            continue
        copy_kib = max(cp)  # the 256 MiB calibration copy is the largest copy dispatch
        pmc[f"{key}_kib_per_step"] = sum(itv) / len(itv)
        pmc[f"{key}_dispatches"] = len(itv)
        pmc[f"{key}_steps_per_dispatch"] = steps_per_dispatch(itr[0]["Kernel_Name"])
        pmc[f"{key}_copy_kib"] = copy_kib
        pmc[f"{key}_scale"] = (COPY_BYTES / 1024.0) / copy_kib
        pmc[f"{key}_command"] = PMC_CMD.format(ctr=ctr, sub=sub)
    if "fetch_scale" in pmc and "write_scale" in pmc:
        fetch = pmc["fetch_kib_per_step"] * pmc["fetch_scale"] * 1024
        write = pmc["write_kib_per_step"] * pmc["write_scale"] * 1024
        SB, TL, TR = step_geometry(1, 8, 32768, 256)
        alg = step_bytes_per_launch(1, 8, 32768, 128, 2, SB, TL, TR)
        lines += ["", "HBM traffic of the fused step (rocprofv3 --pmc, one counter per run):",
                  "  " + pmc["fetch_command"], "  " + pmc["write_command"],
                  f"  FETCH_SIZE {pmc['fetch_kib_per_step']:.0f} KiB/step "
                  f"({pmc['fetch_steps_per_dispatch']} steps per dispatch) x {pmc['fetch_scale']:.3f} "
                  f"(256 MiB copy read {pmc['fetch_copy_kib']:.0f} KiB) = {fetch / 1e6:.1f} MB",
                  f"  WRITE_SIZE {pmc['write_kib_per_step']:.0f} KiB/step x {pmc['write_scale']:.3f} "
                  f"(256 MiB copy wrote {pmc['write_copy_kib']:.0f} KiB) = {write / 1e6:.1f} MB",
                  f"  total {(fetch + write) / 1e6:.1f} MB per step; algorithmic {alg / 1e6:.1f} MB "
                  f"(ratio {(fetch + write) / alg:.3f})",
                  f"  kernel sources hash {pmc['kernel_source_hash']}"]
        with open(PMC_FILE, "w") as f:
            json.dump(pmc, f, indent=1)
    with open(TRACE_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    summarize_sq(d)
    summarize_sweeps(d)
    summarize_l2(d)
    summarize_lds(d)


def _per_kernel(path, names):
    """Counter sums per dispatch, averaged per kernel name, from a rocprofv3
    counter_collection CSV."""
    import glob
    files = glob.glob(os.path.join(path, "*counter_collection.csv"))
    if not files:
        return {}
    per = {}
    for r in _csv_rows(files[0]):
        if r["Counter_Name"] not in names:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        per.setdefault(key, {})
        per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for (k, _), v in per.items():
        acc = out.setdefault(k, {"_n": 0})
        acc["_n"] += 1
        for c, x in v.items():
            acc[c] = acc.get(c, 0.0) + x
    return {k: {c: (x / v["_n"] if c != "_n" else x) for c, x in v.items()} for k, v in out.items()}


def sweep_bytes(name, L=32768, H=8, d=128):
    """HBM floor of one dispatch of an output or backward kernel at the
    long-context workload: every tensor it streams or holds read once, its
    fp32 output written once (bf16 tensors of L d 2 bytes per head)."""
    t16, t32 = H * L * d * 2, H * L * d * 4
    if "output_sweep" in name:
        return 3 * t16 + t32                      # Q, K, V in; O out
    if "bw_rowdot" in name:
        return t16 + t32                          # dO, O in
    if "bw_sweep_kernel" in name:
        mode = int(name.split(",")[2])
        return {0: 2 * t16, 1: 4 * t16 + t32, 2: 4 * t16 + t32}[mode]
    return None


def summarize_sweeps(d):
    """Output and backward kernels: time per dispatch (trace), HBM bytes
    (FETCH_SIZE, WRITE_SIZE, copy-calibrated) and the fraction of the HBM
    floor their time reaches."""
    import glob
    traces = glob.glob(os.path.join(d, "trace", "*kernel_stats.csv"))
    if not traces:  # an LDS probe run only
        summarize_lds(d)
        return
    stats = _csv_rows(traces[0])
    try:
        with open(PMC_FILE) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return
    fetch = _per_kernel(os.path.join(d, "fetch"), {"FETCH_SIZE"})
    write = _per_kernel(os.path.join(d, "write"), {"WRITE_SIZE"})
    lines = ["Output and backward kernels of the long-context workload (B=1, H=8, L=32768, d=128,",
             "W=256, R=2, bf16): time per dispatch from the kernel trace, HBM bytes per dispatch",
             "from FETCH_SIZE and WRITE_SIZE (scaled by the 256 MiB copy calibration), and the",
             "fraction of the kernel's HBM floor (every tensor it reads once, its fp32 output",
             "written once, at 8 TB/s) that its time reaches.", "", HOW,
             "  " + TRACE_CMD, "  " + PMC_CMD.format(ctr="FETCH_SIZE", sub="fetch"),
             "  " + PMC_CMD.format(ctr="WRITE_SIZE", sub="write"), "  " + SUMMARIZE_CMD, "",
             f"{'avg_us':>8} {'fetch_MB':>9} {'write_MB':>9} {'floor_MB':>9} {'floor_us':>9} {'frac':>6}  kernel"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        fb = sweep_bytes(name)
        if fb is None:
            continue
        us = float(r["AverageNs"]) / 1e3
        fm = fetch.get(name, {}).get("FETCH_SIZE")
        wm = write.get(name, {}).get("WRITE_SIZE")
        fms = f"{fm * pmc['fetch_scale'] * 1024 / 1e6:9.1f}" if fm is not None else f"{'-':>9}"
        wms = f"{wm * pmc['write_scale'] * 1024 / 1e6:9.1f}" if wm is not None else f"{'-':>9}"
        floor_us = fb / PEAK_HBM * 1e6
        short = name.split("(")[0].replace("void sinkattn::", "")
        lines.append(f"{us:8.1f} {fms} {wms} {fb / 1e6:9.1f} {floor_us:9.1f} {floor_us / us:6.3f}  {short}")
    lines += ["", f"  kernel sources hash {kernel_source_hash()}"]
    with open(SWEEP_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_l2(d):
    """L2 hit rate and DRAM-bound read requests per kernel (one rocprofv3
    --pmc pass).  TCC_EA0_RDREQ_DRAM counts the L2's read requests to the
    memory controller side; the MI355X Infinity Cache sits behind it and has no
    counter here, so its hits cannot be split from HBM reads."""
    per = _per_kernel(os.path.join(d, "tcc"), set(TCC_COUNTERS.split()))
    if not per:
        return
    lines = ["L2 (TCC) counters per dispatch, long-context workload (B=1, H=8, L=32768, d=128, W=256,",
             "T=100, R=2, bf16); the persistent step kernel's dispatch covers T + R = 102 steps.", "",
             HOW, "  " + TCC_CMD, "  " + SUMMARIZE_CMD, "",
             f"{'hit_rate':>8} {'rdreq_M':>8} {'dram_frac':>9}  kernel"]
    for name, v in sorted(per.items(), key=lambda kv: -kv[1].get("TCC_EA0_RDREQ_sum", 0.0)):
        if "sinkattn" not in name:
            continue
        h, m = v.get("TCC_HIT_sum", 0.0), v.get("TCC_MISS_sum", 0.0)
        rq, dr = v.get("TCC_EA0_RDREQ_sum", 0.0), v.get("TCC_EA0_RDREQ_DRAM_sum", 0.0)
        short = name.split("(")[0].replace("void sinkattn::", "")
        lines.append(f"{h / max(h + m, 1.0):8.3f} {rq / 1e6:8.2f} {dr / max(rq, 1.0):9.3f}  {short}")
    lines += ["", "  hit_rate = TCC_HIT / (TCC_HIT + TCC_MISS); rdreq_M = L2 read requests to the fabric",
              "  (millions per dispatch); dram_frac = TCC_EA0_RDREQ_DRAM / TCC_EA0_RDREQ.",
              f"  kernel sources hash {kernel_source_hash()}"]
    with open(L2_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def lds_probe():
    """Cycles per wave-wide 128-bit LDS read per CU for the step kernel's
    K-tile read pattern at each ring row stride (sinkattn_measure_lds)."""
    import torch

    import entropic_ot_banded_amd as eoba

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    eoba.load_library()
    out = {str(rs): round(eoba.measure_lds(rs, device="cuda:0"), 3) for rs in LDS_STRIDES}
    out["256_xor"] = round(eoba.measure_lds(256, swizzle=True, device="cuda:0"), 3)
    print(json.dumps({"lds_probe": {"cycles_per_read": out, "read_bytes": 1024,
                                    "pattern": "lane (r, g): 16 bytes at 16 g + 64 c of row r, c = 0..3; "
                                               "8 waves x 17 tiles of a 32-tile ring"}}))


def summarize_lds(d):
    """Bank-conflict cycles per LDS instruction of each LDS probe variant
    (one rocprofv3 --pmc pass) beside the cycles per read the same run
    measured."""
    per = {}
    path = os.path.join(d, "lds")
    if not os.path.isdir(path):
        return
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        return
    for r in _csv_rows(files[0]):
        if "lds_probe_kernel" not in r["Kernel_Name"]:
            continue
        key = r["Kernel_Name"].split("lds_probe_kernel<")[1].split(">")[0]
        per.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cyc = {}
    jf = os.path.join(d, "lds_probe.json")
    if os.path.exists(jf):
        with open(jf) as f:
            for line in f:
                if line.startswith("{"):
                    cyc = json.loads(line)["lds_probe"]["cycles_per_read"]
    lines = ["LDS read pattern of the fused step kernel's K-tile operand reads (sinkattn_measure_lds):",
             "one workgroup of 8 waves per CU, each wave reading 17 consecutive tiles of a 32-tile",
             "ring of 16-row tiles per pass; lane (r, g) reads the 16 bytes at 16 g + 64 c of row r",
             "(c = 0..3), one wave-wide 128-bit read = 1024 bytes.", "", HOW, "  " + LDS_CMD,
             "  " + SUMMARIZE_CMD, "",
             f"{'row bytes':>10} {'swizzle':>8} {'cycles/read':>12} {'B/clk/CU':>9} {'conflict cyc/LDS inst':>22}"]
    for key in sorted(per, key=lambda k: (int(k.split(",")[0]), k)):
        rs, swz = key.split(",")[0].strip(), "true" in key
        v = per[key]
        conf = sum(v.get("SQ_LDS_BANK_CONFLICT", [0.0])) / max(sum(v.get("SQ_INSTS_LDS", [1.0])), 1.0)
        c = cyc.get(rs + ("_xor" if swz else ""))
        lines.append(f"{rs:>10} {('xor' if swz else '-'):>8} {c if c is not None else float('nan'):12.2f} "
                     f"{(1024.0 / c) if c else float('nan'):9.1f} {conf:22.2f}")
    lines += ["", "  conflict cyc/LDS inst = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS over the probe's dispatches",
              "  (the ring fill's writes included, under 1% of its LDS instructions); the step kernel",
              "  keeps 272-byte rows (288 would fit only by moving its column partials into the row padding)."]
    with open(LDS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sq(d):
    """Issue counters of the fused step kernel from one rocprofv3 --pmc pass
    (d/sq), per Sinkhorn step, set against the algorithmic work of a step."""
    import glob
    files = glob.glob(os.path.join(d, "sq", "*counter_collection.csv"))
    if not files:
        return
    per = {}
    for r in _csv_rows(files[0]):
        if "iter_kernel" not in r["Kernel_Name"]:
            continue
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
        per.setdefault(key, {})[r["Counter_Name"]] = (per.get(key, {}).get(r["Counter_Name"], 0.0)
                                                      + float(r["Counter_Value"]))
    if not per:
        return
    names = SQ_COUNTERS.split()
    avg = {c: sum(v.get(c, 0.0) / steps_per_dispatch(k[1]) for k, v in per.items()) / len(per) for c in names}
    step_omega = work_counts(1, 8, 32768, 128, 256, 1, 0)[0]  # band entries of one step, all 8 heads
    cycles = avg["GRBM_GUI_ACTIVE"] / 8  # summed over the 8 XCDs
    simds = 256 * 4
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + SQ_COUNTERS + " --output-format csv "
           "-d $OUT/sq -o run -- python3 $REPO/bench.py --steps 2 --warmup 1 " + PROF_ARGS)
    lines = ["Issue counters of the fused step kernel (iter_kernel), long-context workload",
             "(B=1, H=8, L=32768, d=128, W=256, T=100, R=2, bf16), per Sinkhorn step, averaged over "
             f"{len(per)} dispatches:", "", HOW, "  " + cmd, "  " + SUMMARIZE_CMD, ""]
    for c in names:
        lines.append(f"  {c:32s} {avg[c]:16.0f}")
    mfma_busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * simds) if cycles else float("nan")
    flops_hw = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    lines += ["",
              f"  active cycles per step (GRBM_GUI_ACTIVE / 8 XCDs): {cycles:.0f}",
              f"  MFMA pipe busy: {mfma_busy:.3f} of {simds} SIMDs x active cycles",
              f"  bf16 MFMA flops counted: {flops_hw / 1e9:.2f} G per step; algorithmic 2 d |Omega| = "
              f"{2 * 128 * step_omega / 1e9:.2f} G (ratio {flops_hw / (2 * 128 * step_omega):.3f}: tile overcompute)",
              f"  exp (v_exp_f32 and other f32 transcendentals) x 64 lanes: {avg['SQ_INSTS_VALU_TRANS_F32'] * 64 / 1e6:.1f} M "
              f"per step; band entries |Omega| = {step_omega / 1e6:.1f} M",
              f"  VALU instructions per band entry x 64 lanes: {avg['SQ_INSTS_VALU'] * 64 / step_omega:.2f}",
              f"  LDS instructions per step: {avg['SQ_INSTS_LDS'] / 1e6:.2f} M",
              f"  kernel sources hash {kernel_source_hash()}"]
    with open(SQ_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def host_cores() -> int:
    """CPU cores this process may use (the scheduler's affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(prob, heads=None, length=None):
    """The float64 oracle (as is) on a bounded sample of the same workload:
    `heads` of its H independent heads (same input values; default one per
    host core, at most H), all L tokens unless `length` cuts a prefix (then
    with uniform marginals over the prefix), one process per head; scaled to
    whole-workload tokens/s (the work is linear in L and in H)."""
    import numpy as np

    import oracle
    import workloads

    cores = host_cores()
    if heads is None:
        heads = max(1, min(prob.H, cores, 16))
    procs = min(heads, cores)
    sub = workloads.make(5, heads=list(range(heads)), R=prob.R)
    Ls = sub.L if length is None else min(length, sub.L)
    sl = lambda x: np.ascontiguousarray(x[:, :, :Ls])
    a = np.full((sub.B, Ls), 1.0 / Ls, dtype=np.float32)
    t0 = time.perf_counter()
    oracle.forward_backward_batch(sl(sub.Q), sl(sub.K), sl(sub.V), a, a.copy(), sub.W, sub.T, sub.R,
                                  sl(sub.dO), processes=procs)
    dt = time.perf_counter() - t0
    # the metric counts a token once for all H heads: the whole workload
    # (B L tokens, H heads) takes dt * (H / heads) * (L / Ls)
    value = prob.B * prob.L / (dt * (prob.H / heads) * (prob.L / Ls))
    return {"value": value, "unit": "tokens/s", "cores": procs, "kind": "oracle",
            "sample": f"first {Ls} of {prob.L} tokens of {heads} of {prob.H} heads (independent problems) "
                      f"of the same inputs, uniform marginals over the sample, full T={sub.T}, R={sub.R}, "
                      f"forward+backward, float64 numpy/scipy, {procs} processes (one head each) on "
                      f"{cores} host cores: {dt:.1f} s; scaled to the whole workload (work is linear in L and in H)",
            "seconds": dt}


def time_workload(eoba, torch, prob, steps, warmup, dev, tensors=None):
    """Mean ms of one forward + backward of `prob` (inputs resident on the
    device; `tensors` = (Q, K, V, dO) already there), HIP events on the
    current stream around `steps` back-to-back steps after `warmup` untimed
    ones."""
    import numpy as np

    dt = torch.bfloat16 if prob.dtype == "bf16" else torch.float32
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt).contiguous()  # noqa: E731
    Q, K, V, dO = tensors if tensors is not None else (up(prob.Q), up(prob.K), up(prob.V), up(prob.dO))
    a = torch.from_numpy(prob.a).to(dev)
    b = torch.from_numpy(prob.b).to(dev)
    ln = None if prob.lengths is None else torch.from_numpy(prob.lengths.astype(np.int32)).to(dev)
    ws = None

    def step():
        nonlocal ws
        O, _, _, ws = eoba.forward(Q, K, V, prob.W, prob.T, prob.R, a, b, ln, prob.dustbin, workspace=ws)
        eoba.backward(Q, K, V, prob.W, prob.T, prob.R, a, b, O, dO, ws, ln, prob.dustbin)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / steps


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 20 untimed steps first: the step time falls by about 2% over the first
    # ten or so steps of a process (the clocks settling under load), and the
    # line reports the steady state
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--R", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the MFMA/exp peak probes")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="heads in the oracle sample (default: one per host core, at most H and 16)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR", help="write profiles/ summaries from rocprofv3 CSV output")
    ap.add_argument("--converge-tol", type=float, default=5e-5,
                    help="also time the early-stopping base at this tolerance (0: skip)")
    ap.add_argument("--converge-every", type=int, default=5)
    ap.add_argument("--certificate-rmax", type=int, default=4,
                    help="also time the stop-gradient bias certificate up to this depth (0: skip)")
    ap.add_argument("--certificate-tau", type=float, default=1e-5)
    ap.add_argument("--contraction-block", type=int, default=128,
                    help="also time the projective contraction diagnostic at this block size (0: skip)")
    ap.add_argument("--r4-steps", type=int, default=5,
                    help="also time the same workload with the R=4 tail over this many steps (0: skip)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the step times of the tiny, mid, protein-like and dustbin workloads")
    ap.add_argument("--lds-probe", action="store_true",
                    help="only measure the LDS read pattern of the step kernel at each ring row stride")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.lds_probe:
        lds_probe()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each (batch, head) problem is independent, so a batch would shard across "
              "GPUs by head with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import entropic_ot_banded_amd as eoba
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    eoba.load_library()
    dev = torch.device("cuda:0")
    prob = workloads.make(5, R=args.R)
    W, T, R = prob.W, prob.T, prob.R
    dt = torch.bfloat16 if prob.dtype == "bf16" else torch.float32

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt).contiguous()

    Q, K, V, dO = up(prob.Q), up(prob.K), up(prob.V), up(prob.dO)
    a = torch.from_numpy(prob.a).to(dev)
    b = torch.from_numpy(prob.b).to(dev)
    ws = None

    def step():
        nonlocal ws
        O, u, v, ws = eoba.forward(Q, K, V, W, T, R, a, b, workspace=ws)
        dQ, dK, dV, _ = eoba.backward(Q, K, V, W, T, R, a, b, O, dO, ws)
        return O, dQ

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    # forward / backward split: events between the launches of every timed
    # step, on the same stream (the host enqueues ahead, so the stream runs
    # back to back and each bracket is device time)
    fb = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step_split(e3):
        nonlocal ws
        e3[0].record(stream)
        O, u, v, ws = eoba.forward(Q, K, V, W, T, R, a, b, workspace=ws)
        e3[1].record(stream)
        dQ, dK, dV, _ = eoba.backward(Q, K, V, W, T, R, a, b, O, dO, ws)
        e3[2].record(stream)
        return O, dQ

    eoba.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        O, dQ = step_split(fb[i])
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev[0].elapsed_time(ev[1])
    iter_ms, iter_launches = eoba.timing_collect()
    eoba.timing_enable(False)
    if not (torch.isfinite(O).all() and torch.isfinite(dQ).all()):
        raise RuntimeError("non-finite output")
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in fb) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in fb) / args.steps

    # The convergence-controlled base on the same inputs, T as its cap
    # (sinkattn_forward_converge; host-timed, since it waits at each check).
    converged = None
    if args.converge_tol > 0:
        def conv_step():
            O, u, v, wsc, T_used, err_last = eoba.forward_converge(
                Q, K, V, W, T, R, a, b, args.converge_tol, args.converge_every, workspace=ws)
            eoba.backward(Q, K, V, W, T_used, R, a, b, O, dO, wsc)
            return T_used, err_last
        conv_step()
        times = []
        for _ in range(5):
            torch.cuda.synchronize()
            c0 = time.perf_counter()
            T_used, err_last = conv_step()
            torch.cuda.synchronize()
            times.append(time.perf_counter() - c0)
        c_ms = sorted(times)[len(times) // 2] * 1e3
        converged = {"tol": args.converge_tol, "check_every": args.converge_every, "T_max": T,
                     "T_used": T_used, "err_last": err_last, "ms_per_step": round(c_ms, 4),
                     "tokens_per_s": round(prob.real_tokens() / (c_ms * 1e-3), 1),
                     "timing": "host clock, median of 5 forward_converge + backward"}

    # Stop-gradient bias certificate: a forward keeping R_max tail steps, then
    # eta_R for R = 0..R_max (one backward pass of depth R_max, then the dQ/dK sweeps of
    # every shallower depth) and the selected depth.
    certificate = None
    if args.certificate_rmax > 0:
        Rm = args.certificate_rmax
        Oc, _, _, wsc = eoba.forward(Q, K, V, W, T, Rm, a, b)
        eoba.tail_certificate(Q, K, V, W, T, Rm, a, b, Oc, dO, wsc, tau=args.certificate_tau)  # warm
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        _, _, _, eta, r_sel = eoba.tail_certificate(Q, K, V, W, T, Rm, a, b, Oc, dO, wsc, tau=args.certificate_tau)
        torch.cuda.synchronize()
        c_ms = (time.perf_counter() - c0) * 1e3
        certificate = {"T": T, "R_max": Rm, "eta": [float(f"{x:.4e}") for x in eta],
                       "tau": args.certificate_tau,
                       "selected_R": r_sel,
                       "ms": round(c_ms, 3), "timing": "host clock, one call (a depth-R_max backward and R_max dQ/dK sweep pairs)"}
        del Oc, wsc

    # Projective contraction diagnostic over the diagonal band blocks.
    contraction = None
    if args.contraction_block > 0:
        blk = args.contraction_block
        eoba.block_contraction(Q, K, W, blk)  # warm
        cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        cev[0].record(stream)
        delta, kappa = eoba.block_contraction(Q, K, W, blk)
        cev[1].record(stream)
        torch.cuda.synchronize()
        contraction = {"block": blk, "blocks": int(kappa.numel()), "delta_max": round(float(delta.max()), 4),
                       "kappa_max": round(float(kappa.max()), 4), "kappa_mean": round(float(kappa.mean()), 4),
                       "ms": round(cev[0].elapsed_time(cev[1]), 4)}

    # The same inputs with the R = 4 tail (the comparison run of the
    # long-context workload): step time, throughput and the whole path's
    # MFMA/exp fraction counted per half-step.
    r4 = None
    if args.r4_steps > 0 and R != 4:
        p4 = workloads.make(5, R=4)
        ms4 = time_workload(eoba, torch, p4, args.r4_steps, 2, dev, tensors=(Q, K, V, dO))
        _, _, _, f4, x4 = work_counts(prob.B, prob.H, prob.L, prob.d, W, T, 4)
        t4 = ms4 * 1e-3
        r4 = {"R": 4, "ms_per_step": round(ms4, 4), "tokens_per_s": round(prob.real_tokens() / t4, 1),
              "flops": f4, "exps": x4, "frac": round(max(f4 / PEAK_MFMA[prob.dtype], x4 / PEAK_EXP) / t4, 4),
              "steps": args.r4_steps}
        del p4

    # Step times of the other workloads (latency-bound at these sizes; the
    # dustbin one takes per-step launches with its own kernel between them).
    others = {}
    if not args.no_other_configs:
        for key, cfg, dtyp in (("tiny", 1, None), ("mid", 2, None), ("mid_bf16", 2, "bf16"),
                               ("protein", 3, None), ("dustbin", 4, None)):
            pc = workloads.make(cfg, dtype=dtyp)
            msc = time_workload(eoba, torch, pc, 20, 3, dev)
            others[key] = {"shape": list(pc.shape), "W": pc.W, "T": pc.T, "R": pc.R, "dtype": pc.dtype,
                           "dustbin": pc.dustbin, "ms_per_step": round(msc, 4),
                           "tokens_per_s": round(pc.real_tokens() / (msc * 1e-3), 1)}

    if args.copy_calibration:
        x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()

    # Sustained bf16 MFMA and v_exp_f32 rates on this GPU (after the timed
    # region): the roofline fractions are also given against these.
    peaks = eoba.measure_peaks(dev) if prob.dtype == "bf16" and not args.no_peaks else None

    ms_per_step = ms_total / args.steps
    tokens = prob.real_tokens()
    value = tokens / (ms_per_step * 1e-3)
    omega, ex_flops, ex_exps, sv_flops, sv_exps = work_counts(prob.B, prob.H, prob.L, prob.d, W, T, R)
    peak = PEAK_MFMA[prob.dtype]
    # Dominant kernel: the fused Sinkhorn step (T + R steps per forward, all in
    # one persistent launch), timed with HIP events around its launch on the
    # stream it runs on.  Its roofline counts the work per half-step: the row
    # and the column update each take a score contraction (2 d flops) and an
    # exp per band entry, so 4 d flops and 2 exps per entry per Sinkhorn step
    # (this kernel evaluates each score once per step and reuses it for both
    # updates), against the published bf16 MFMA and v_exp_f32 peaks.
    avg_step_s = (iter_ms / iter_launches) * 1e-3 if iter_launches else float("nan")
    launch_steps = T + R
    step_flops = omega * 4 * prob.d
    step_exps = omega * 2
    t_roof = max(step_flops / peak, step_exps / PEAK_EXP)
    traffic = load_pmc()  # HBM bytes per Sinkhorn step (rocprofv3 counters), or None
    roofline = {"bound": "mfma" if step_flops / peak >= step_exps / PEAK_EXP else "exp",
                "achieved": round(step_flops * launch_steps / (avg_step_s * launch_steps) / 1e12, 2),
                "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(t_roof / avg_step_s, 4),
                "traffic": None if traffic is None else round(traffic * launch_steps / 1e9, 3),
                "traffic_unit": "GB per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": "iter_kernel (fused Sinkhorn step; persistent: T + R steps per launch)",
                "launch_us": round(avg_step_s * launch_steps * 1e6, 2), "steps_per_launch": launch_steps,
                "avg_step_us": round(avg_step_s * 1e6, 3), "steps_timed": iter_launches,
                "flops_per_launch": step_flops * launch_steps, "exps_per_launch": step_exps * launch_steps,
                "exp_frac": round(step_exps / avg_step_s / PEAK_EXP, 4),
                "executed_mfma_frac": round(omega * 2 * prob.d / avg_step_s / peak, 4)}
    # the same kernel against its own HBM traffic model (Q and K streamed once
    # per step, potentials and column partials): a separate figure
    esize = 2 if prob.dtype == "bf16" else 4
    SB, TL, TR = step_geometry(prob.B, prob.H, prob.L, W)
    step_bytes = step_bytes_per_launch(prob.B, prob.H, prob.L, prob.d, esize, SB, TL, TR)
    design_hbm = {"bytes_per_step": int(step_bytes), "achieved": round(step_bytes / avg_step_s / 1e9, 1),
                  "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(step_bytes / avg_step_s / PEAK_HBM, 4),
                  "traffic_per_step": None if traffic is None else round(traffic / 1e9, 4)}
    t_s = ms_per_step * 1e-3
    path = {"executed": {"flops": ex_flops, "exps": ex_exps,
                         "frac": round(max(ex_flops / peak, ex_exps / PEAK_EXP) / t_s, 4)},
            "half_step_counting": {"flops": sv_flops, "exps": sv_exps,
                                "frac": round(max(sv_flops / peak, sv_exps / PEAK_EXP) / t_s, 4)},
            "peak_mfma_flops": peak, "peak_exp_per_s": PEAK_EXP}
    if peaks is not None:
        pm, pe = peaks["mfma_bf16_flops"], peaks["exp_per_s"]
        roofline["frac_measured_peaks"] = round(max(step_flops / pm, step_exps / pe) / avg_step_s, 4)
        path["executed"]["frac_measured"] = round(max(ex_flops / pm, ex_exps / pe) / t_s, 4)
        path["half_step_counting"]["frac_measured"] = round(max(sv_flops / pm, sv_exps / pe) / t_s, 4)
        path["measured_peaks"] = {"mfma_bf16_flops": float(f"{pm:.4g}"), "exp_per_s": float(f"{pe:.4g}"),
                                  "clock_ghz": round(peaks["clock_hz"] / 1e9, 3),
                                  "probe": "sinkattn_measure_peaks: v_mfma_f32_16x16x32_bf16 and v_exp_f32 "
                                           "issue rates with every CU loaded"}
    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": prob.dtype, "data": "synthetic",
           "config": {"workload": "long-context banded Sinkhorn attention, forward + exact R-tail backward",
                      "B": prob.B, "H": prob.H, "L": prob.L, "d": prob.d, "W": W, "T": T, "R": R,
                      "inputs": "bf16", "accumulate": "fp32", "state": "fp64"},
           "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "wall_s": round(wall, 3),
           "roofline": roofline, "design_hbm": design_hbm, "path_roofline": path}
    if r4 is not None:
        out["r4"] = r4
    if others:
        out["other_workloads"] = others
    if converged is not None:
        out["converged_base"] = converged
    if certificate is not None:
        out["certificate"] = certificate
    if contraction is not None:
        out["contraction"] = contraction
    if not args.no_cpu_baseline:
        cb = cpu_baseline(prob, args.cpu_heads)
        cb.pop("seconds", None)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
