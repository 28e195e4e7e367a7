#!/usr/bin/env python3
"""Benchmark of the low-rank bottleneck block on one MI355X.

One step = one forward (with the rank-r checkpoint) + one backward of the block
over one batch of synthetic, seeded input already resident in HBM, through the
C ABI (the shard workload "btp_shard" times its two seam calls instead; the
workload "lowrank_mlp" times the per-projection low-rank SwiGLU MLP).  Prints
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
METRIC_MLP = "per-projection low-rank SwiGLU MLP fwd+bwd TFLOP/s (bf16) and % MFMA peak; tokens/s"
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


def split_tiles(T, d, r, g, n_up, dn, dtype="bf16") -> int:
    """Tiles the library's weight-gradient plan splits over two token halves
    when the 256 x 256 tiles fill between one and two rounds of the 256 CUs (the
    rest run whole); 0 when that plan does not apply.  dn: the dB width."""
    if dtype != "bf16":
        return 0
    cd = lambda a, b: -(-a // b)
    tiles_b = n_up * cd(r, 256) * cd(dn, 256)
    tiles = tiles_b + cd(d, 256) * cd(g * r, 256)
    S = 512 - tiles
    ok = (tiles > 256 and 0 < S <= tiles_b and tiles - S <= 256 and (tiles - S) % 8 == 0 and (2 * S) % 8 == 0
          and cd(T, 64) >= 32)
    return S if ok else 0


def wgrad_split_tiles(wl) -> int:
    return split_tiles(wl.T, wl.d, wl.r, wl.g, wl.n_up, wl.d, wl.dtype)


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
    if name == "up":   # the residual variant also reads residual_i
        return 2.0 * T * r * d * nu, e * (T * r * nu + nu * r * d + nu * T * d * (2 if wl.residual else 1))
    if name == "dz":
        return 2.0 * T * d * r * nu, e * (nu * T * d + nu * r * d + T * gr + T * gr + T * zcols) + 4 * T
    if name == "wgrad":
        return (2.0 * T * r * d * nu + 2.0 * T * d * gr,
                e * (T * (zcols or gr) + nu * T * d + T * d + T * gr + d * gr) + 4 * (d * gr + nu * r * d))
    if name == "wgrad_reduce":   # the split-K sum: only its fp32 results count
        split = wgrad_split_tiles(wl)
        if split:   # only the split (dB) tiles are summed; dgamma from the dA tiles' row partials
            return 0.0, 4 * split * 256 * 256 + 4 * d * (-(-gr // 256) * 2 + 1)
        return 0.0, 4 * (d * gr + nu * r * d)
    if name == "sum_parts":   # dgamma from the whole dA tiles' row partials
        return 0.0, 4 * d * (-(-gr // 256) * 2 + 1)
    if name == "dx":   # the residual variant also reads the residual path's gradient
        return 2.0 * T * gr * d, e * (T * gr + d * gr + (3 if wl.residual else 2) * T * d) + 4 * T
    if name == "fold_gamma":   # the one-kernel small-rank path also reorders B
        return 0.0, e * (2 * d * gr + d + (2 * nu * r * d if one_kernel_forward(wl) else 0))
    if name == "rms_stats":
        return 0.0, e * T * d + 4 * T
    if name == "finish":
        return 0.0, 4 * (T * gr + T) + e * (T * gr + T * zcols)
    return 0.0, 0.0


def mlp_kernel_work(wl, name: str):
    """Algorithmic (flops, HBM bytes) of all launches of kernel `name` in one
    step of the per-projection MLP (forward, then a backward that recomputes
    gate, up and s): each launch's operands read once and results written once;
    GEMM flops as executed, the recomputation included."""
    T, d, f, r = wl.T, wl.d, wl.f, wl.r
    e = 2 if wl.dtype == "bf16" else 4
    res = 1 if wl.residual else 0
    if name == "up":   # gate, up (+s), out; then gate and up (+s) again in the backward
        fl = 2.0 * T * r * (4 * f + d)
        gate = e * (T * r + r * f + T * f)
        upf = e * (T * r + r * f + 2 * T * f)
        return fl, gate + upf + e * (T * r + r * d + (1 + res) * T * d) + gate + upf + e * T * f
    if name == "down":   # x . A_in (normalised), s . A_o (plain)
        return 2.0 * T * r * (2 * d + f), e * (T * d + 2 * d * r + 2 * T * r + T * f + f * r + T * r) + 4 * T
    if name == "dz":     # dout . B_o^T; (dgate, dup) . (B_g, B_u)^T with the S' partials
        return (2.0 * T * r * (d + 2 * f),
                e * (T * d + r * d + 2 * T * r + 2 * T * f + 2 * r * f + 2 * T * 2 * r) + 4 * T)
    if name == "wgrad":  # dB_o, dA_o; dB_g, dB_u, dA_in
        return (2.0 * T * r * (d + f) + 2.0 * T * r * (2 * f + 2 * d),
                e * (T * r + T * d + T * f + T * r) + 4 * (r * d + f * r)
                + e * (2 * T * r + 2 * T * f + T * d + 2 * T * r + 2 * d * r) + 4 * (2 * r * f + 2 * d * r))
    if name == "dx":     # ds with the SwiGLU backward (gate, up in; dgate, dup out); dx with RMSNorm
        return (2.0 * T * r * (f + 2 * d),
                e * (T * r + f * r + 4 * T * f) + e * (2 * T * r + 2 * d * r + (2 + res) * T * d) + 4 * T)
    if name == "fold_gamma":
        return 0.0, e * (2 * d * 2 * r + d)
    if name == "wgrad_reduce":   # each layer's reduction, where its plan has one
        def red(dA_rows, g, n_up, dn, gamma):
            cd = lambda a, b: -(-a // b)
            tiles = n_up * cd(r, 256) * cd(dn, 256) + cd(dA_rows, 256) * cd(g * r, 256)
            if tiles <= 256 and 8 * tiles >= 7 * 256:   # one token pass
                return 0
            st = split_tiles(T, dA_rows, r, g, n_up, dn, wl.dtype)
            if st:
                return 4 * st * 256 * 256 + (4 * dA_rows * (cd(g * r, 256) * 2 + 1) if gamma else 0)
            return 4 * (n_up * r * dn + dA_rows * g * r)
        return 0.0, red(f, 1, 1, d, False) + red(d, 2, 2, f, True)
    return 0.0, 0.0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def checkpoint_bytes(wl) -> dict:
    """What the backward keeps per block: the rank-r pre-activation h (and the
    4-byte-a-token RMSNorm statistic), against keeping the normalised input,
    h and z as a plain autograd graph of the block would."""
    e = 2 if wl.dtype == "bf16" else 4
    gr = wl.g * wl.r
    zc = wl.r if wl.act == "swiglu" else (0 if wl.act == "identity" else gr)
    kept = e * wl.T * gr + 4 * wl.T
    plain = e * wl.T * (wl.d + gr + zc)
    return {"h_bytes": e * wl.T * gr, "rstd_bytes": 4 * wl.T, "kept_bytes": kept,
            "xn_h_z_bytes": plain, "ratio": plain / kept}


def cpu_baseline(wl, inp, budget_s: float = 24.0):
    """The oracle as it stands (NumPy) on the host cores: float64 (the
    correctness oracle) and the same code in float32, each timed for the
    forward and for forward + backward, on a bounded sample of the workload's
    tokens (the first rows of `inp`, the same seeded draw the GPU ran on; all of
    them when they fit the budget).  `value` is the float64 leg of the step the
    GPU figure times, in the metric's unit."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    is_mlp = hasattr(wl, "f")
    fwd_step = not is_mlp and (wl.seam or wl.fwd_only)

    def oracle_pass(rows, with_bwd):
        x = inp.x.v[:rows]
        if is_mlp:
            w = [t.v for t in (inp.gamma, inp.A_in, inp.B_g, inp.B_u, inp.A_o, inp.B_o)]
            oracle.mlp_fwd(x, *w, wl.r, wl.eps, residual=x if wl.residual else None)
            if with_bwd:
                dout = inp.dout.v[:rows]
                oracle.mlp_bwd(x, *w, dout, wl.r, wl.eps, dx_residual=dout if wl.residual else None)
            return
        args = (x, inp.gamma.v, inp.A.v, [b.v for b in inp.B])
        if wl.seam:
            p, ss = oracle.down_partial(*args[:3])
            oracle.up_finish(p, ss, args[3], wl.r, wl.g, wl.act, wl.eps, wl.D)
            return
        oracle.block_fwd(*args, wl.r, wl.g, wl.act, wl.eps, wl.D, residual=[x] if wl.residual else None)
        if with_bwd:
            dy = [t.v[:rows] for t in inp.dy]
            oracle.block_bwd(*args, dy, wl.r, wl.g, wl.act, wl.eps, wl.D,
                             dx_residual=dy[0] if wl.residual else None)

    def timed(rows, with_bwd, prec, reps=1):
        with oracle.working_precision(prec):
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle_pass(rows, with_bwd)
            return time.perf_counter() - t0

    # legs: (precision, with backward, share of the budget)
    legs = [("f64", False, 0.15), ("f32", False, 0.1)]
    if not fwd_step:
        legs = [("f64", True, 0.45), ("f64", False, 0.15), ("f32", True, 0.25), ("f32", False, 0.15)]
    probe = min(wl.T, 256)
    out = {}
    for prec, with_bwd, share in legs:
        dt = np.float64 if prec == "f64" else np.float32
        tp = timed(probe, with_bwd, dt)
        leg_budget = budget_s * share
        rows = int(min(wl.T, max(probe, probe * leg_budget / max(tp, 1e-3))))
        rows = max(probe, rows // 64 * 64) if rows < wl.T else wl.T
        total, passes = timed(rows, with_bwd, dt), 1
        # a whole-workload sample that ends well inside its share is repeated on
        # the same inputs until the share is spent; t is per pass
        if rows == wl.T and total < leg_budget / 2:
            more = min(int(leg_budget / total) - 1, 50)
            total += timed(rows, with_bwd, dt, more)
            passes += more
        t = total / passes
        sub = wl.replace(T=rows)
        flops = sub.fwd_flops() + (sub.bwd_flops() if with_bwd else 0.0)
        key = f"{prec}_{'fwd_bwd' if with_bwd else 'fwd'}"
        out[key] = {"tflops": flops / t / 1e12, "tokens_per_s": rows / t, "s_per_pass": t, "rows": rows,
                    "passes": passes,
                    "fwd_gbs": sub.fwd_bytes() / t / 1e9 if not (with_bwd or is_mlp) else None}
        log(f"cpu oracle {key}: {rows} rows, {passes} pass(es), {t:.3f} s per pass")
    main = out["f64_fwd" if fwd_step else "f64_fwd_bwd"]
    rows = main["rows"]
    what = (f"first {rows} of {wl.T} tokens" if rows < wl.T else
            f"all {wl.T} tokens, {main['passes']} pass{'es' if main['passes'] > 1 else ''}")
    step = "forward" if fwd_step else "fwd+bwd"
    sample = (f"{what}, seed 0, the float64 NumPy oracle's {step}, {main['s_per_pass']:.2f} s per pass; "
              f"legs: float64 and float32, forward and fwd+bwd, each on its own row sample")
    res = {"unit": "TFLOP/s", "value": main["tflops"], "cores": int(threads), "kind": "oracle", "sample": sample,
           "tokens_per_s": main["tokens_per_s"], "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
           "legs": out}
    if not is_mlp and wl.fwd_only and wl.hbm_metric:
        res["unit"], res["value"] = "GB/s", main["fwd_gbs"]
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: about %.2f s of steps, at least 20)" % TIMED_S)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: about %.1f s of steps, at least 20)" % WARM_S)
    ap.add_argument("--workload", default="qkv_silu_ckpt")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=24.0, help="seconds of oracle work on the host")
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
    from workloads import MLP_WORKLOADS, WORKLOADS, make_inputs, make_mlp_inputs

    def dev(t):
        if t.dtype == "bf16":
            return torch.from_numpy(t.store.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(t.store).cuda()

    torch.cuda.set_device(0)
    if args.workload in MLP_WORKLOADS:
        return main_mlp(args, MLP_WORKLOADS[args.workload], rb, torch, dev, make_mlp_inputs)
    wl = WORKLOADS[args.workload]
    log("workload", wl)
    inp = make_inputs(wl, seed=0, with_dy=not (wl.seam or wl.fwd_only))

    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    dy = None if (wl.seam or wl.fwd_only) else [dev(t) for t in inp.dy]
    if args.no_cpu_baseline:
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

        if wl.residual:   # the sublayer out = x + block(x): residual add and dy -> dx fused
            def step():
                rb.lr_block_fwd_residual(dims, x, gamma, A, B, [x], y, h, rstd, wsf)
                rb.lr_block_bwd_residual(dims, x, gamma, A, B, h, rstd, dy, dy[0], dx, dgamma, dA, dB, wsb)
        else:
            def step():
                rb.lr_block_fwd_rstd(dims, x, gamma, A, B, y, h, rstd, wsf)
                rb.lr_block_bwd_rstd(dims, x, gamma, A, B, h, rstd, dy, dx, dgamma, dA, dB, wsb)
        flops = wl.fwd_flops() + wl.bwd_flops()

    ms_step, per_kernel, dominant, dom_ms = measure(args, step, rb, torch)
    roof = roofline(wl, dominant, dom_ms, kernel_work(wl, dominant), wl.dtype)
    tflops = flops / (ms_step * 1e-3) / 1e12

    metric, value, unit = METRIC, tflops, "TFLOP/s"
    if wl.fwd_only and wl.hbm_metric:
        metric, value, unit = METRIC_FWD, wl.fwd_bytes() / (ms_step * 1e-3) / 1e9, "GB/s"
    elif wl.fwd_only:
        metric = "low-rank block forward TFLOP/s (bf16)"
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
           "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "r": wl.r, "g": wl.g, "act": wl.act,
                      "d_norm": wl.D, "residual": wl.residual,
                      "step": "seam fwd" if wl.seam else ("fwd" if wl.fwd_only else "fwd+bwd"),
                      "parallelism": "none (1 GPU)"},
           "tflops": tflops,
           "tokens_per_s": wl.T / (ms_step * 1e-3),
           "pct_mfma_peak": 100.0 * tflops / PEAK_TFLOPS[wl.dtype],
           "kernel_ms_warmup_step": per_kernel,
           "checkpoint": None if (wl.seam or wl.fwd_only) else checkpoint_bytes(wl),
           "roofline": roof}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def main_mlp(args, wl, rb, torch, dev, make_mlp_inputs):
    """The per-projection low-rank SwiGLU MLP: one step = lr_mlp_fwd (keeping
    h_in, h_out and rstd) + lr_mlp_bwd, as the sublayer out = x + mlp(x) when
    the workload has the residual."""
    log("workload", wl)
    inp = make_mlp_inputs(wl, seed=0)
    x = dev(inp.x)
    w = [dev(t) for t in (inp.gamma, inp.A_in, inp.B_g, inp.B_u, inp.A_o, inp.B_o)]
    dout = dev(inp.dout)
    if args.no_cpu_baseline:
        del inp
    dims = rb.make_mlp_dims(wl.T, wl.d, wl.f, wl.r, wl.dtype, wl.eps)
    dt = rb.TORCH_DTYPE[dims.dtype]
    f32 = dict(dtype=torch.float32, device="cuda")
    out_t = torch.empty((wl.T, wl.d), dtype=dt, device="cuda")
    h_in = torch.empty((wl.T, 2 * wl.r), dtype=dt, device="cuda")
    h_out = torch.empty((wl.T, wl.r), dtype=dt, device="cuda")
    rstd = torch.empty(wl.T, **f32)
    dx = torch.empty((wl.T, wl.d), dtype=dt, device="cuda")
    grads = [torch.empty(wl.d, **f32), torch.empty((wl.d, 2 * wl.r), **f32), torch.empty((wl.r, wl.f), **f32),
             torch.empty((wl.r, wl.f), **f32), torch.empty((wl.f, wl.r), **f32), torch.empty((wl.r, wl.d), **f32)]
    wsf, wsb = rb.mlp_workspace(dims, False), rb.mlp_workspace(dims, True)
    res = x if wl.residual else None
    dres = dout if wl.residual else None

    def step():
        rb.lr_mlp_fwd(dims, x, *w, res, out_t, h_in, h_out, rstd, wsf)
        rb.lr_mlp_bwd(dims, x, *w, h_in, h_out, rstd, dout, dres, dx, *grads, wsb)

    ms_step, per_kernel, dominant, dom_ms = measure(args, step, rb, torch)
    roof = roofline(wl, dominant, dom_ms, mlp_kernel_work(wl, dominant), wl.dtype)
    flops = wl.fwd_flops() + wl.bwd_flops()
    tflops = flops / (ms_step * 1e-3) / 1e12
    e = 2 if wl.dtype == "bf16" else 4
    out = {"metric": METRIC_MLP, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
           "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "f": wl.f, "r": wl.r, "residual": wl.residual,
                      "step": "fwd+bwd", "parallelism": "none (1 GPU)"},
           "tflops": tflops,
           "tflops_with_recompute": (flops + wl.recompute_flops()) / (ms_step * 1e-3) / 1e12,
           "tokens_per_s": wl.T / (ms_step * 1e-3),
           "pct_mfma_peak": 100.0 * tflops / PEAK_TFLOPS[wl.dtype],
           "kernel_ms_warmup_step": per_kernel,
           "checkpoint": {"kept_bytes": e * wl.T * 3 * wl.r + 4 * wl.T,
                          "wide_bytes": e * wl.T * 3 * wl.f,
                          "ratio": (e * wl.T * 3 * wl.f) / (e * wl.T * 3 * wl.r + 4 * wl.T)},
           "roofline": roof}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def measure(args, step, rb, torch):
    """Warm-up, a traced warm-up step (per-kernel times, the dominant kernel),
    then the timed region.  Returns (ms per step, per-kernel ms of the traced
    step, the dominant kernel's name, its ms per timed step for the traced
    steps)."""
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
    per_kernel, per_count = {}, {}
    for i in range(rb.lr_trace_count()):
        name, ms = rb.lr_trace_elapsed(i)
        per_kernel[name] = per_kernel.get(name, 0.0) + ms
        per_count[name] = per_count.get(name, 0) + 1
    rb.lr_trace_end()
    torch.cuda.synchronize()
    dominant = max(per_kernel, key=per_kernel.get)
    log("warm-up kernel ms:", {k: round(v, 4) for k, v in per_kernel.items()}, "dominant:", dominant)

    # timed region: K steps; the dominant kernel's launches of the first TRACED
    # steps are bracketed by HIP events on its stream.  Each event pair leaves
    # the GPU idle for a few microseconds, so bracketing every launch would
    # inflate the step time that the headline value comes from.
    traced = max(1, min(args.steps, 5))
    per_step = per_count[dominant]
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rb.lr_trace_begin(dominant, traced * per_step)
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
    # the dominant kernel's time per step (the sum of its launches in a step)
    dom_step = float(np.sum(dom_ms)) / (len(dom_ms) / per_step) if dom_ms else float("nan")
    return ms_step, per_kernel, dominant, (dom_step, per_step)


def roofline(wl, dominant, dom, work, dtype):
    """Roofline of the dominant kernel: its algorithmic flops (or bytes) per step
    over its time per step (for a kernel launched once per step, per launch)."""
    dom_avg, per_step = dom
    kf, kb = work
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (PEAK_GBS * 1e9)
    if kf > 0 and kf / max(kb, 1) > ridge:
        roof = {"bound": "mfma", "achieved": kf / (dom_avg * 1e-3) / 1e12, "peak": PEAK_TFLOPS[dtype],
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kb / (dom_avg * 1e-3) / 1e9, "peak": PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dominant
    roof["kernel_ms"] = dom_avg
    roof["launches_per_step"] = per_step
    roof["algorithmic_flops"] = kf
    roof["algorithmic_bytes"] = kb
    roof["traffic"] = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        rec = json.load(open(tpath)).get(f"{wl.name}/{dominant}")
        if rec and rec.get("source_hash") == source_hash():
            # per step like `achieved` (per launch for a kernel launched once a step)
            roof["traffic"] = rec.get("bytes_per_step", rec["bytes_per_launch"])
    return roof


if __name__ == "__main__":
    main()
