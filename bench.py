#!/usr/bin/env python3
"""Benchmark: forward + backward banded Sinkhorn attention on one MI355X.

Workload (the long-context configuration): B=1, H=8, L=32768, d=128, band
W=256 (offsets [-128, 127]), T=100 stopped base steps, R=2 tail steps,
uniform marginals, Q, K, V ~ N(0,1)/sqrt(d) and dO ~ N(0,1) rounded to
bf16 (seeded synthetic data); fp32 accumulation, fp64 Sinkhorn state.

One step = sinkattn_forward + sinkattn_backward over the whole batch (every
row of the hot path), inputs resident in HBM.  Prints ONE JSON line with the
throughput, the roofline of the dominant kernel (the fused Sinkhorn step,
timed per launch with HIP events on its stream) and the float64 oracle timed
on the host's cores on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--R 2] [--no-cpu-baseline]
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
PMC_FILE = os.path.join(ROOT, "profiles", "iter_kernel_long_context_pmc.json")
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
    Survey counting: one score per half-step, 2(T+R) 2d + 4d forward and
    (4R+10) d backward; 2(T+R) + 1 + 2R + 1 exps.
    """
    omega = B * H * band_entries_fast(L, W)
    ex_flops = omega * ((T + R) * 2 * d + 4 * d + 4 * d + (2 * R - 1) * 2 * d + 12 * d)
    ex_exps = omega * ((T + R) + 1 + 1 + (2 * R - 1) + 2)
    sv_flops = omega * (2 * (T + R) * 2 * d + 4 * d + (4 * R + 10) * d)
    sv_exps = omega * (2 * (T + R) + 1 + 2 * R + 1)
    return omega, ex_flops, ex_exps, sv_flops, sv_exps


def load_pmc(launch_units):
    """HBM traffic per launch of the fused step from committed rocprofv3
    counters, scaled by a copy-kernel calibration; None if absent or taken
    on different kernel sources."""
    try:
        with open(PMC_FILE) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    if pmc.get("kernel_source_hash") != kernel_source_hash():
        return None
    fetch = pmc["fetch_kib_per_dispatch"] * pmc["fetch_scale"]
    write = pmc["write_kib_per_dispatch"] * pmc["write_scale"]
    return (fetch + write) * 1024.0


def cpu_baseline(prob, heads):
    """The float64 oracle (as is) on `heads` of the H independent heads,
    single process; scaled to whole-workload tokens/s."""
    import oracle
    import workloads

    sub = workloads.make(5, heads=list(range(heads)), R=prob.R)
    t0 = time.perf_counter()
    oracle.forward_backward_batch(sub.Q, sub.K, sub.V, sub.a, sub.b, sub.W, sub.T, sub.R, sub.dO,
                                  processes=1)
    dt = time.perf_counter() - t0
    tokens = prob.B * prob.L
    value = tokens * heads / prob.H / dt
    return {"value": value, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} of {prob.H} heads (independent problems) of the same workload, "
                      f"full T={prob.T}, R={prob.R}, forward+backward, float64 numpy/scipy, "
                      f"1 process; {dt:.1f} s, scaled by H/{heads}",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--R", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=1, help="heads in the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
    eoba.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(args.steps):
        O, dQ = step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev[0].elapsed_time(ev[1])
    iter_ms, iter_launches = eoba.timing_collect()
    eoba.timing_enable(False)
    if not (torch.isfinite(O).all() and torch.isfinite(dQ).all()):
        raise RuntimeError("non-finite output")

    # separate forward / backward split (untimed region for the main value)
    fb = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fb[0].record(stream)
    O, u, v, ws = eoba.forward(Q, K, V, W, T, R, a, b, workspace=ws)
    fb[1].record(stream)
    eoba.backward(Q, K, V, W, T, R, a, b, O, dO, ws)
    fb[2].record(stream)
    torch.cuda.synchronize()
    fwd_ms, bwd_ms = fb[0].elapsed_time(fb[1]), fb[1].elapsed_time(fb[2])

    if args.copy_calibration:
        x = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()

    ms_per_step = ms_total / args.steps
    tokens = prob.real_tokens()
    value = tokens / (ms_per_step * 1e-3)
    omega, ex_flops, ex_exps, sv_flops, sv_exps = work_counts(prob.B, prob.H, prob.L, prob.d, W, T, R)
    peak = PEAK_MFMA[prob.dtype]
    # dominant kernel: the fused Sinkhorn step, 2d flops per band entry per launch
    avg_launch_s = (iter_ms / iter_launches) * 1e-3 if iter_launches else float("nan")
    launch_flops = omega * 2 * prob.d
    achieved = launch_flops / avg_launch_s / 1e12
    traffic = load_pmc(omega)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved * 1e12 / peak, 4),
                "traffic": None if traffic is None else round(traffic / 1e9, 4),
                "kernel": "iter_kernel (fused Sinkhorn step)",
                "avg_launch_us": round(avg_launch_s * 1e6, 3), "launches": iter_launches,
                "flops_per_launch": launch_flops,
                "traffic_unit": "GB per launch",
                "exp_frac": round(omega / avg_launch_s / PEAK_EXP, 4)}
    t_s = ms_per_step * 1e-3
    path = {"executed": {"flops": ex_flops, "exps": ex_exps,
                         "frac": round(max(ex_flops / peak, ex_exps / PEAK_EXP) / t_s, 4)},
            "survey_counting": {"flops": sv_flops, "exps": sv_exps,
                                "frac": round(max(sv_flops / peak, sv_exps / PEAK_EXP) / t_s, 4)},
            "peak_exp_per_s": PEAK_EXP}
    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": prob.dtype, "data": "synthetic",
           "config": {"workload": "long-context banded Sinkhorn attention, forward + exact R-tail backward",
                      "B": prob.B, "H": prob.H, "L": prob.L, "d": prob.d, "W": W, "T": T, "R": R,
                      "inputs": "bf16", "accumulate": "fp32", "state": "fp64"},
           "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "wall_s": round(wall, 3),
           "roofline": roofline, "path_roofline": path}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(prob, args.cpu_heads)
        cb.pop("seconds", None)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
