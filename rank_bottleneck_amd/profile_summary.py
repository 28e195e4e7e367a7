"""Summaries of rocprofv3 output for this library's kernels.

    python -m rank_bottleneck_amd.profile_summary stats  <kernel_stats.csv> <out.md> --title T --command C
    python -m rank_bottleneck_amd.profile_summary traffic <fetch_counter_collection.csv> <write_counter_collection.csv>
           --workload W --out profiles/traffic.json --command C
    python -m rank_bottleneck_amd.profile_summary mfma <counter_collection.csv> <out.md> --title T --command C

`mfma` summarises one `--pmc MfmaUtil MfmaFlopsBF16` pass per kernel (per launch
position within a step for a kernel launched several times a step): the MFMA
busy fraction (MFMA busy cycles over active cycles times SIMDs), the bf16 MFMA
FLOPs the hardware counted (MFMA ops x 512), the rate those FLOPs give over the
dispatch's duration, and the shader clock that rate and busy fraction imply
(1024 SIMDs x 1024 dense bf16 FLOP per clock each at full MFMA occupancy).

`traffic` converts FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel into
HBM bytes per launch.  Each counter is scaled by the factor that makes the same
counter read exactly right for the plain 256 MiB copy that
`bench.py --copy-calibration` runs first (read 256 MiB, write 256 MiB), and the
entry records a hash of the kernel sources so that stale figures are ignored.
A kernel name launched n times a step (the per-projection MLP launches "up"
five times, with different shapes) is summarised per launch position: the
steps repeat one launch sequence, so position i of a step is every n-th
dispatch of that name from the i-th on; each position's median over the
steps is taken and the positions are added (bytes_per_step), and
bytes_per_launch is that sum over n.  A name launched once a step reduces to
the median over its dispatches.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["rank_bottleneck_amd/csrc/lr_kernels.hip", "rank_bottleneck_amd/csrc/lr_device.h",
                  "rank_bottleneck_amd/csrc/lr_kernels.h", "rank_bottleneck_amd/csrc/lr_pipe.h",
                  "rank_bottleneck_amd/csrc/lr_fused.hip"]
COPY_BYTES = 256 << 20
SHORT = [("k_fused_fwd", "fused"), ("k_fold_fused", "fold_gamma"), ("k_wgrad_sk_reduce", "wgrad_reduce"), ("k_wgrad_reduce", "wgrad_reduce"), ("k_wgrad", "wgrad"), ("k_down", "down"), ("k_up", "up"),
         ("k_dz", "dz"), ("k_dx", "dx"), ("k_rms_stats", "rms_stats"), ("k_fold_gamma", "fold_gamma"),
         ("k_sum_parts", "sum_parts"), ("k_finish", "finish")]


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    k = kernel.replace("_ZN2lr", "")
    for needle, short in SHORT:
        if needle[2:] in k:
            return short
    return kernel


def stats(csv_path: str, out: str, title: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    with open(out, "w") as f:
        f.write(f"# {title}\n\nCommand (repository root, one MI355X):\n\n```\n{command}\n```\n\n")
        f.write("| kernel | name | calls | average us | share % |\n|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {short_name(r['Name'])} | `{r['Name'][:70]}` | {r['Calls']} | "
                    f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |\n")


def _per_kernel(csv_path: str, counter: str):
    """{kernel name: counter values in dispatch order}"""
    rows = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    vals = defaultdict(list)
    for _, k, v in sorted(rows):
        vals[k].append(v)
    return vals


def _per_short(vals):
    """{short name: values in dispatch order} over this library's kernels"""
    out = defaultdict(list)
    for k, v in vals.items():
        if short_name(k) != k:
            out[short_name(k)].extend(v)
    return out


def _per_short_ordered(csv_path: str, counter: str):
    rows = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and short_name(r["Kernel_Name"]) != r["Kernel_Name"]:
            rows.append((int(r["Dispatch_Id"]), short_name(r["Kernel_Name"]), float(r["Counter_Value"])))
    out = defaultdict(list)
    for _, k, v in sorted(rows):
        out[k].append(v)
    return out


def _per_step(values, steps: int) -> float:
    """sum over launch positions of each position's median over the steps"""
    n = max(1, len(values) // steps)
    return sum(statistics.median(values[i::n]) for i in range(n)), n


def traffic(fetch_csv: str, write_csv: str, workload: str, out: str, command: str) -> dict:
    fetch, write = _per_kernel(fetch_csv, "FETCH_SIZE"), _per_kernel(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy:
        raise SystemExit("no calibration copy kernel in the fetch run")
    ck = max(copy, key=lambda k: max(fetch[k]))
    f_scale = COPY_BYTES / (max(fetch[ck]) * 1024.0)
    w_scale = COPY_BYTES / (max(write[ck]) * 1024.0)
    rec = json.load(open(out)) if os.path.exists(out) else {}
    h = source_hash()
    summary = {}
    sf, sw = _per_short_ordered(fetch_csv, "FETCH_SIZE"), _per_short_ordered(write_csv, "WRITE_SIZE")
    steps = min(len(v) for v in sf.values())   # a name launched once a step sets the step count
    for name in sf:
        fpos, n = _per_step(sf[name], steps)
        wpos, _ = _per_step(sw.get(name, [0.0] * len(sf[name])), steps)
        fb, wb = fpos * 1024.0 * f_scale, wpos * 1024.0 * w_scale
        rec[f"{workload}/{name}"] = {"bytes_per_launch": (fb + wb) / n, "bytes_per_step": fb + wb,
                                     "launches_per_step": n, "fetch_bytes": fb / n, "write_bytes": wb / n,
                                     "fetch_scale": f_scale, "write_scale": w_scale, "source_hash": h,
                                     "command": command}
        summary[name] = (fb, wb)
    json.dump(rec, open(out, "w"), indent=1, sort_keys=True)
    return summary


def mfma(csv_path: str, out: str, title: str, command: str) -> None:
    # per short name, in dispatch order; a name launched n times a step is
    # reported per launch position (name#1 .. name#n), as in `traffic`
    rows = []
    for r in csv.DictReader(open(csv_path)):
        k = short_name(r["Kernel_Name"])
        if k == r["Kernel_Name"]:
            continue
        rows.append((int(r["Dispatch_Id"]), k, r["Counter_Name"], float(r["Counter_Value"]),
                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9))
    seq = defaultdict(list)   # name -> [(dispatch, {counter: value}, duration)]
    by_disp = {}
    for disp, k, cname, v, t in sorted(rows):
        if disp not in by_disp:
            by_disp[disp] = (k, {}, t)
            seq[k].append(by_disp[disp])
        by_disp[disp][1][cname] = v
    steps = min(len(v) for v in seq.values()) if seq else 1
    util, flops, dur = defaultdict(list), defaultdict(list), defaultdict(list)
    for k, items in seq.items():
        n = max(1, len(items) // steps)
        for i, (_, vals, t) in enumerate(items):
            key = k if n == 1 else f"{k}#{i % n + 1}"
            if "MfmaUtil" in vals:
                util[key].append(vals["MfmaUtil"])
                dur[key].append(t)
            if "MfmaFlopsBF16" in vals:
                flops[key].append(vals["MfmaFlopsBF16"])
    with open(out, "w") as f:
        f.write(f"# {title}\n\nCommand (repository root, one MI355X):\n\n```\n{command}\n```\n\n")
        f.write("Medians over the profiled launches (kernels run one at a time under counter collection).\n\n")
        f.write("| kernel | MFMA util % | bf16 MFMA GFLOP / launch | duration us | TFLOP/s | % of 2.5 PF | implied clock GHz |\n")
        f.write("|---|---|---|---|---|---|---|\n")
        for k in sorted(util, key=lambda k: -statistics.median(dur[k])):
            u, t = statistics.median(util[k]), statistics.median(dur[k])
            fl = statistics.median(flops[k]) if flops.get(k) else 0.0
            rate = fl / t / 1e12 if t > 0 else 0.0
            clk = rate * 1e12 / (1024 * 1024 * (u / 100.0)) / 1e9 if u > 0 else 0.0
            f.write(f"| {k} | {u:.1f} | {fl / 1e9:.2f} | {t * 1e6:.1f} | {rate:.0f} | {100 * rate / 2500:.1f} | "
                    f"{clk:.2f} |\n")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["stats", "traffic", "mfma"])
    ap.add_argument("inputs", nargs="+")
    ap.add_argument("--title", default="kernel statistics")
    ap.add_argument("--command", default="")
    ap.add_argument("--workload", default="")
    ap.add_argument("--out", default="")
    a = ap.parse_args()
    if a.mode == "stats":
        stats(a.inputs[0], a.inputs[1], a.title, a.command)
    elif a.mode == "mfma":
        mfma(a.inputs[0], a.inputs[1], a.title, a.command)
    else:
        s = traffic(a.inputs[0], a.inputs[1], a.workload, a.out, a.command)
        for k, (fb, wb) in sorted(s.items()):
            print(f"{k:14s} fetch {fb / 1e6:10.1f} MB  write {wb / 1e6:10.1f} MB")
