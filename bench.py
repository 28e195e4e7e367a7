#!/usr/bin/env python3
"""Benchmark of the low-rank bottleneck block on one MI355X.

One step = one forward (with the rank-r checkpoint) + one backward of the block
over one batch of synthetic, seeded input already resident in HBM, through the
C ABI (the shard workload "btp_shard" times its two seam calls instead).  Prints
ONE JSON line: block fwd+bwd TFLOP/s (algorithmic GEMM FLOPs, elementwise work
not counted), tokens/s, % of the bf16 MFMA peak, the roofline of the dominant
kernel (timed with HIP events on its launch stream over the timed region) and
the CPU oracle timed on a bounded row sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "low-rank block fwd+bwd TFLOP/s (bf16) and % MFMA peak; tokens/s per block"
METRIC_FWD = "low-rank block forward HBM GB/s (small-rank, memory-bound sweep)"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA (published)
PEAK_GBS = 8000.0                                # MI355X HBM3E (published)
WARM_S = 0.5     # default untimed warm-up, seconds of steps
TIMED_S = 0.25   # default timed region, seconds of steps
KERNEL_SOURCES = ["rank_bottleneck_amd/csrc/lr_kernels.hip", "rank_bottleneck_amd/csrc/lr_device.h",
                  "rank_bottleneck_amd/csrc/lr_kernels.h", "rank_bottleneck_amd/csrc/lr_pipe.h",
                  "rank_bottleneck_amd/csrc/lr_fused.hip"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def one_kernel_forward(wl) -> bool:
    """Whether the library runs this workload's forward as its one-kernel
    small-rank path (the shapes it documents for that path)."""
    if wl.dtype != "bf16" or wl.seam:
        return False
    if wl.act == "swiglu":
        return wl.g == 2 and wl.r in (64, 128)
    return (wl.r == 64 and wl.g <= 4) or (wl.r == 128 and wl.g <= 2) or (wl.r == 256 and wl.g == 1)


def kernel_work(wl, name: str):
    """Algorithmic (flops, HBM bytes) of one launch of kernel `name`: every
    operand read once and every result written once; GEMM flops only."""
    T, d, r, g, nu = wl.T, wl.d, wl.r, wl.g, wl.n_up
    e = 2 if wl.dtype == "bf16" else 4
    gr = g * r
    zcols = 0 if wl.act == "identity" else (r if wl.act == "swiglu" else gr)
    if name == "down":
        if wl.seam:   # fp32 partial + sumsq
            return 2.0 * T * d * gr, e * (T * d + d * gr) + 4 * (T * gr + T)
        return 2.0 * T * d * gr, e * (T * d + d * gr + T * gr + T * zcols)
    if name == "fused":   # one-kernel small-rank forward: x, A'^T, B, y and h, each once
        return (2.0 * T * d * gr + 2.0 * T * r * d * nu,
                e * (T * d + d * gr + nu * r * d + nu * T * d + T * gr))
    if name == "up":
        return 2.0 * T * r * d * nu, e * (T * r * nu + nu * r * d + nu * T * d)
    if name == "dz":
        return 2.0 * T * d * r * nu, e * (nu * T * d + nu * r * d + T * gr + T * gr + T * zcols) + 4 * T
    if name == "wgrad":
        return (2.0 * T * r * d * nu + 2.0 * T * d * gr,
                e * (T * (zcols or gr) + nu * T * d + T * d + T * gr + d * gr) + 4 * (d * gr + nu * r * d))
    if name == "wgrad_reduce":   # the split-K sum: only its fp32 results count
        return 0.0, 4 * (d * gr + nu * r * d)
    if name == "dx":
        return 2.0 * T * gr * d, e * (T * gr + d * gr + 2 * T * d) + 4 * T
    if name == "fold_gamma":   # the one-kernel small-rank path also reorders B
        return 0.0, e * (2 * d * gr + d + (2 * nu * r * d if one_kernel_forward(wl) else 0))
    if name == "rms_stats":
        return 0.0, e * T * d + 4 * T
    if name == "finish":
        return 0.0, 4 * (T * gr + T) + e * (T * gr + T * zcols)
    return 0.0, 0.0


def cpu_baseline(wl, budget_s: float = 15.0):
    """The oracle (float64 NumPy, as it stands) on a row sample of the same
    workload, on the host cores; reported in the metric's unit."""
    import oracle
    from workloads import make_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def oracle_pass(inp):
        args = (inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B])
        if wl.seam:
            p, ss = oracle.down_partial(*args[:3])
            oracle.up_finish(p, ss, args[3], wl.r, wl.g, wl.act, wl.eps, wl.D)
        elif wl.fwd_only:
            oracle.block_fwd(*args, wl.r, wl.g, wl.act, wl.eps, wl.D)
        else:
            oracle.block_fwd(*args, wl.r, wl.g, wl.act, wl.eps, wl.D)
            oracle.block_bwd(*args, [t.v for t in inp.dy], wl.r, wl.g, wl.act, wl.eps, wl.D)

    def run(inp, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle_pass(inp)
        return time.perf_counter() - t0

    probe = min(wl.T, 256)
    tp = run(make_inputs(wl, seed=0, rows=probe))
    rows = int(min(wl.T, max(probe, probe * budget_s / max(tp, 1e-3))))
    rows = max(probe, rows // 64 * 64) if rows < wl.T else wl.T
    log(f"cpu oracle: probe {probe} rows {tp:.2f}s -> sample {rows} rows")
    inp = make_inputs(wl, seed=0, rows=rows)
    total, passes = run(inp), 1
    # a sample that is the whole workload and ends well inside the budget is
    # repeated on the same inputs until the budget is spent; t is per pass
    if rows == wl.T and total < budget_s / 2:
        more = min(int(budget_s / total) - 1, 50)
        total += run(inp, more)
        passes += more
    t = total / passes
    what = (f"first {rows} of {wl.T} tokens" if rows < wl.T else
            f"all {wl.T} tokens, {passes} pass{'es' if passes > 1 else ''}")
    sub = wl.replace(T=rows)
    if wl.fwd_only and wl.hbm_metric:
        return {"value": sub.fwd_bytes() / t / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{what}, seed 0, float64 NumPy forward, {t:.2f} s per pass ({total:.1f} s)",
                "tokens_per_s": rows / t}
    flops = sub.fwd_flops() + (0 if (wl.seam or wl.fwd_only) else sub.bwd_flops())
    step = "forward" if (wl.seam or wl.fwd_only) else "fwd+bwd"
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}, seed 0, float64 NumPy {step}, {t:.2f} s per pass ({total:.1f} s)",
            "tokens_per_s": rows / t}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: about %.2f s of steps, at least 20)" % TIMED_S)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: about %.1f s of steps, at least 20)" % WARM_S)
    ap.add_argument("--workload", default="qkv_identity")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work on the host")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the steps, copy a 256 MiB buffer once (a plain copy kernel of known size, "
                         "used to scale the HBM byte counters of a profiling run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the block's hot path runs on one GPU's shard and this build has no "
              "multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_bottleneck_amd as rb
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    log("workload", wl)
    torch.cuda.set_device(0)
    inp = make_inputs(wl, seed=0, with_dy=not (wl.seam or wl.fwd_only))

    def dev(t):
        if t.dtype == "bf16":
            return torch.from_numpy(t.store.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(t.store).cuda()

    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    dy = None if (wl.seam or wl.fwd_only) else [dev(t) for t in inp.dy]
    del inp
    dims = rb.make_dims(wl.T, wl.d, wl.r, wl.g, wl.act, wl.dtype, wl.eps, wl.d_norm)
    dt = rb.TORCH_DTYPE[dims.dtype]
    gr, nu = wl.g * wl.r, wl.n_up
    y = [torch.empty((wl.T, wl.d), dtype=dt, device="cuda") for _ in range(nu)]
    h = torch.empty((wl.T, gr), dtype=dt, device="cuda")
    wsf = rb.workspace(dims, False)
    if wl.seam:
        partial = torch.empty((wl.T, gr), dtype=torch.float32, device="cuda")
        sumsq = torch.empty(wl.T, dtype=torch.float32, device="cuda")

        def step():
            rb.lr_down_partial(dims, x, gamma, A, partial, sumsq, wsf)
            rb.lr_up_finish(dims, partial, sumsq, B, y, h, wsf)
        flops = wl.fwd_flops()
    elif wl.fwd_only:
        def step():
            rb.lr_block_fwd(dims, x, gamma, A, B, y, h, wsf)
        flops = wl.fwd_flops()
    else:
        wsb = rb.workspace(dims, True)
        dx = torch.empty((wl.T, wl.d), dtype=dt, device="cuda")
        dgamma = torch.empty(wl.d, dtype=torch.float32, device="cuda")
        dA = torch.empty((wl.d, gr), dtype=torch.float32, device="cuda")
        dB = [torch.empty((wl.r, wl.d), dtype=torch.float32, device="cuda") for _ in range(nu)]
        rstd = torch.empty(wl.T, dtype=torch.float32, device="cuda")  # kept with h for the backward

        def step():
            rb.lr_block_fwd_rstd(dims, x, gamma, A, B, y, h, rstd, wsf)
            rb.lr_block_bwd_rstd(dims, x, gamma, A, B, h, rstd, dy, dx, dgamma, dA, dB, wsb)
        flops = wl.fwd_flops() + wl.bwd_flops()

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Default step counts follow time: the GPU raises its clocks over the first
    # tens of milliseconds of sustained work (a 20-step run after 5 warm-up steps
    # measured ~10% below the steady rate), so the untimed warm-up lasts about
    # WARM_S and the timed region about TIMED_S.  The calibration (one step for
    # first-call costs, then three timed on the host clock) counts as warm-up.
    done = 0
    if args.warmup is None or args.steps is None:
        step()
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        per = (time.perf_counter() - c0) / 3
        done = 4
        if args.warmup is None:
            args.warmup = max(20, math.ceil(WARM_S / per))
        if args.steps is None:
            args.steps = max(20, math.ceil(TIMED_S / per))
    # warm-up; the last warm-up step is traced per kernel to find the dominant one
    for i in range(max(args.warmup - done - 1, 0)):
        step()
    args.warmup = done + max(args.warmup - done - 1, 0) + 1
    rb.lr_trace_begin(None, 64)
    step()
    per_kernel = {}
    for i in range(rb.lr_trace_count()):
        name, ms = rb.lr_trace_elapsed(i)
        per_kernel[name] = per_kernel.get(name, 0.0) + ms
    rb.lr_trace_end()
    torch.cuda.synchronize()
    dominant = max(per_kernel, key=per_kernel.get)
    log("warm-up kernel ms:", {k: round(v, 4) for k, v in per_kernel.items()}, "dominant:", dominant)

    # timed region: K steps; the dominant kernel's first TRACED launches are
    # bracketed by HIP events on its stream.  Each event pair leaves the GPU idle
    # for a few microseconds, so bracketing every launch would inflate the step
    # time that the headline value comes from.
    traced = max(1, min(args.steps, 5))
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rb.lr_trace_begin(dominant, traced)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    dom_ms = [rb.lr_trace_elapsed(i)[1] for i in range(rb.lr_trace_count())]
    rb.lr_trace_end()
    ms_step = t0.elapsed_time(t1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step (wall {wall:.3f} s)")

    tflops = flops / (ms_step * 1e-3) / 1e12
    dom_avg = float(np.mean(dom_ms)) if dom_ms else float("nan")
    kf, kb = kernel_work(wl, dominant)
    ridge = PEAK_TFLOPS[wl.dtype] * 1e12 / (PEAK_GBS * 1e9)
    if kf > 0 and kf / max(kb, 1) > ridge:
        roof = {"bound": "mfma", "achieved": kf / (dom_avg * 1e-3) / 1e12, "peak": PEAK_TFLOPS[wl.dtype],
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kb / (dom_avg * 1e-3) / 1e9, "peak": PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dominant
    roof["kernel_ms"] = dom_avg
    roof["algorithmic_flops"] = kf
    roof["algorithmic_bytes"] = kb
    roof["traffic"] = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        rec = json.load(open(tpath)).get(f"{wl.name}/{dominant}")
        if rec and rec.get("source_hash") == source_hash():
            roof["traffic"] = rec["bytes_per_launch"]

    metric, value, unit = METRIC, tflops, "TFLOP/s"
    if wl.fwd_only and wl.hbm_metric:
        metric, value, unit = METRIC_FWD, wl.fwd_bytes() / (ms_step * 1e-3) / 1e9, "GB/s"
    elif wl.fwd_only:
        metric = "low-rank block forward TFLOP/s (bf16)"
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
           "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "r": wl.r, "g": wl.g, "act": wl.act,
                      "d_norm": wl.D, "step": "seam fwd" if wl.seam else ("fwd" if wl.fwd_only else "fwd+bwd"),
                      "parallelism": "none (1 GPU)"},
           "tflops": tflops,
           "tokens_per_s": wl.T / (ms_step * 1e-3),
           "pct_mfma_peak": 100.0 * tflops / PEAK_TFLOPS[wl.dtype],
           "kernel_ms_warmup_step": per_kernel,
           "roofline": roof}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
