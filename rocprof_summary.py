#!/usr/bin/env python3
"""Summaries of rocprofv3 output for profiles/ (text only).

The GPU commands run bench.py under rocprofv3 and write CSV into a results
folder; this turns one folder (or several) into the short markdown (and, for
HBM traffic, JSON) kept under profiles/.  It reads CSV and the bench JSON
line only, and runs nothing on the GPU.

    python rocprof_summary.py trace    DIR  --config NAME --bench JSON --command CMD [--cold N]
    python rocprof_summary.py traffic  FETCH_DIR WRITE_DIR --config NAME --command CMD --command CMD --json OUT
    python rocprof_summary.py counters DIR [DIR ...] --config NAME --command CMD [--command CMD ...]

The attention kernel is the one bench.py rates: decode_valu_kernel,
decode_mfma_kernel, prefill_kernel or copy_blocks_kernel, plus reduce_kernel
when the context is split (the two make the attention).  Figures are per
dispatch: averages over dispatches for durations, medians for counters.
"""

from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MAIN_KERNELS = ("decode_valu_kernel", "decode_mfma_kernel", "prefill_kernel", "copy_blocks_kernel")
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# rocprofv3 derived metrics: the expressions its counter list gives on gfx950
EXPRESSIONS = {
    "MfmaUtil": "100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMDs)",
    "VALUBusy": "100 * sum(SQ_ACTIVE_INST_VALU) / CUs / max(GRBM_GUI_ACTIVE)",
    "SALUBusy": "100 * sum(SQ_INST_CYCLES_SALU) / CUs / max(GRBM_GUI_ACTIVE)",
    "OccupancyPercent": "400 * sum(SQ_WAVE_CYCLES) / max(GRBM_GUI_ACTIVE) / CUs / 32 (resident waves, % of 32 per CU)",
    "LdsUtil": "100 * sum(SQ_LDS_IDX_ACTIVE) / (max(GRBM_GUI_ACTIVE) * CUs)",
    "LdsBankConflict": "sum(SQ_LDS_BANK_CONFLICT) / (sum(SQ_LDS_IDX_ACTIVE) - sum(SQ_LDS_BANK_CONFLICT))",
    "TCC_HIT_sum": "L2 hits, all channels",
    "TCC_MISS_sum": "L2 misses, all channels",
    "MfmaFlopsBF16": "512 * SQ_INSTS_VALU_MFMA_MOPS_BF16",
}


def read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def is_main(name: str) -> bool:
    return (name.startswith("void pa::") or name.startswith("pa::")) and any(k in name for k in MAIN_KERNELS)


def is_reduce(name: str) -> bool:  # pa_reduce's kernel (not a framework reduction of the same name)
    return "pa::" in name and "reduce_kernel" in name


def short(name: str, n: int = 110) -> str:
    return name if len(name) <= n else name[:n]


def trace(args):
    rows = read_csv(os.path.join(args.dirs[0], "run_kernel_trace.csv"))
    stats = read_csv(os.path.join(args.dirs[0], "run_kernel_stats.csv"))
    bench = json.load(open(args.bench)) if args.bench else None
    per = {}
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    main = [k for k in per if is_main(k)]
    red = [k for k in per if is_reduce(k)]
    out = [f"# Kernel trace: {args.config}", "", "Commands (repository root, one MI355X):", "", "```"]
    out += [c for c in args.command] + ["```", "", "`--stats` summary (run_kernel_stats.csv), durations in microseconds:", "",
                                        "| kernel | calls | average | min | max | share |", "|---|---|---|---|---|---|"]
    for s in stats:
        out.append(f"| `{short(s['Name'])}` | {s['Calls']} | {float(s['AverageNs']) / 1e3:.2f} | "
                   f"{float(s['MinNs']) / 1e3:.2f} | {float(s['MaxNs']) / 1e3:.2f} | {float(s['Percentage']):.1f}% |")
    out.append("")
    # bench.py's launches, in order: the settle steps (the GPU leaving its idle clocks), the
    # warm-up steps, the timed passes, then the cold launches (each after a 512 MiB read):
    # warm figures are taken over the launches after the settle and warm-up, cold ones over
    # the cold launches
    skip = int(bench.get("settle_steps", 0)) + int(bench.get("warmup", 0)) if bench else 0
    # (the count bench.py reports, else --cold)
    n_cold = int((bench or {}).get("breakdown_us", {}).get("cold_launches", args.cold))
    total_avg = 0.0
    total_cold = 0.0
    for k in main + red:
        d = per[k]
        warm = d[skip:len(d) - n_cold] or d
        avg = statistics.fmean(warm)
        total_avg += avg
        out.append(f"`{short(k)}`: {len(d)} launches; after the {skip} settle and warm-up steps and before the "
                   f"{n_cold} cold launches, {len(warm)} warm launches: average {avg:.2f} us, median "
                   f"{statistics.median(warm):.2f} us.")
        if n_cold:
            cold = d[-n_cold:]
            total_cold += statistics.fmean(cold)
            if not is_reduce(k):
                out.append(f"  The last {n_cold} launches are bench.py's cold launches (each after a 512 MiB read): "
                           f"average {statistics.fmean(cold):.2f} us, median {statistics.median(cold):.2f} us.")
    if bench is not None:
        r = bench.get("roofline", {})
        out.append("")
        out.append(f"Same command's JSON line: roofline over {r.get('timing', 'the timed launches')}: "
                   f"avg_launch_us {r.get('avg_launch_us')}, achieved {r.get('achieved')} {r.get('unit')} = "
                   f"{100 * float(r.get('frac', 0)):.1f}% of peak; ms_per_step {bench.get('ms_per_step')}, "
                   f"value {bench.get('value')} {bench.get('unit')}.")
        if r.get("unit") == "GB/s" and main and "algorithmic_bytes_per_launch" in r:
            b = float(r["algorithmic_bytes_per_launch"])
            base = total_avg
            if n_cold and r.get("timing", "").startswith("cold"):
                base = total_cold
            out.append(f"Trace-based rate: {b:.0f} algorithmic bytes / {base:.2f} us = {b / base / 1e3:.1f} GB/s = "
                       f"{100 * b / base / 1e3 / HBM_PEAK_GBPS:.1f}% of 8 TB/s"
                       + (" (attention kernel + pa_reduce)" if red else "") + ".")
        elif r.get("unit") == "TFLOP/s" and main and "algorithmic_flops_per_launch" in r:
            fl = float(r["algorithmic_flops_per_launch"])
            out.append(f"Trace-based rate: {fl:.4g} FLOP / {total_avg:.2f} us = {fl / total_avg / 1e6:.1f} TFLOP/s = "
                       f"{100 * fl / total_avg / 1e6 / MFMA_BF16_PEAK_TFLOPS:.1f}% of the bf16 matrix peak.")
    print("\n".join(out))


CALIBRATION_COPIES = 5  # bench.py --calibrate-copy: 1 GiB device-to-device copies at the end of the run


def per_dispatch(d):
    """{(kernel, counter): {dispatch id: value}} of a counter-collection folder."""
    rows = read_csv(os.path.join(d, "run_counter_collection.csv"))
    per = {}
    for r in rows:
        per.setdefault((r["Kernel_Name"], r["Counter_Name"]), {}).setdefault(int(r["Dispatch_Id"]), 0.0)
        per[(r["Kernel_Name"], r["Counter_Name"])][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return per


def counters_of(d):
    per = per_dispatch(d)
    return {k: statistics.median(v.values()) for k, v in per.items()}, {k: len(v) for k, v in per.items()}


def traffic(args):
    import bench
    import workloads as wl

    fetch, nf = counters_of(args.dirs[0])
    write, nw = counters_of(args.dirs[1])
    cal = {}
    for d in list(args.dirs[:2]) + list(args.calibration):  # calibration copies: the runs' own, or others'
        for (k, c), v in per_dispatch(d).items():
            if "copyBuffer" in k and c in ("FETCH_SIZE", "WRITE_SIZE") and c not in cal:
                # bench.py --calibrate-copy makes five 1 GiB copies in a row; other copies (the
                # workload's pools placed on the device, results read back) come singly or in
                # pairs, of other sizes: take the largest run of five consecutive copy
                # dispatches that agree to 1%
                vals = [v[i] for i in sorted(v)]
                runs = [vals[i:i + CALIBRATION_COPIES] for i in range(len(vals) - CALIBRATION_COPIES + 1)]
                runs = [r for r in runs if min(r) > 0 and max(r) <= 1.01 * min(r)]
                if runs:
                    cal[c] = statistics.median(max(runs, key=statistics.median))
    moved_kib = (1 << 30) / 1024
    fs = moved_kib / cal["FETCH_SIZE"] if cal.get("FETCH_SIZE") else 1.0
    ws = moved_kib / cal["WRITE_SIZE"] if cal.get("WRITE_SIZE") else 1.0
    kernels = [k for (k, c) in fetch if c == "FETCH_SIZE" and (is_main(k) or is_reduce(k))]
    copy = args.config == "copy-blocks"
    if copy:  # pa_copy_blocks: the bytes the bench line names (every block read once and written once)
        p = None
        alg = int(json.load(open(args.bench))["roofline"]["algorithmic_bytes_per_launch"])
        sources = bench.COPY_SOURCES
    else:
        p = wl.make_problem(args.config)
        ab = wl.algorithmic_bytes(p)
        alg = ab["kv_unique"] + ab["q"] + (ab["out"] if p.query_start is not None else 0)  # prefill: + the output
        sources = bench.PREFILL_SOURCES if p.query_start is not None else bench.KERNEL_SOURCES
    fetch_b = sum(fetch[(k, "FETCH_SIZE")] for k in kernels) * 1024 * fs
    write_b = sum(write.get((k, "WRITE_SIZE"), 0.0) for k in kernels) * 1024 * ws
    res = {
        "workload": args.config,
        "kernels": kernels,
        "kernel_source_sha": bench.kernel_source_hash(sources),
        "fetch_bytes_per_launch": round(fetch_b),
        "write_bytes_per_launch": round(write_b),
        "fetch_size_kib_raw": {k: fetch[(k, "FETCH_SIZE")] for k in kernels},
        "write_size_kib_raw": {k: write.get((k, "WRITE_SIZE"), 0.0) for k in kernels},
        "copy_calibration": {"bytes_each_way": 1 << 30, "fetch_size_kib": cal.get("FETCH_SIZE"),
                             "write_size_kib": cal.get("WRITE_SIZE"), "fetch_scale": fs, "write_scale": ws},
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": (fetch_b + write_b) / alg,
        "commands": args.command,
    }
    with open(args.json, "w") as f:
        json.dump(res, f, indent=1)
    out = [f"# HBM traffic: {args.config}", "", "Commands (repository root, one MI355X), one counter per run:", "",
           "```"] + args.command + ["```", "",
                                    f"Calibration: bench.py --calibrate-copy copies 1 GiB device to device; FETCH_SIZE "
                                    f"reads {cal.get('FETCH_SIZE')} KiB and WRITE_SIZE {cal.get('WRITE_SIZE')} KiB for "
                                    f"it against {moved_kib:.0f} KiB moved each way: scale factors {fs:.4f} (fetch) and "
                                    f"{ws:.4f} (write).", ""]
    for k in kernels:
        out.append(f"`{short(k)}` ({nf[(k, 'FETCH_SIZE')]} dispatches): FETCH_SIZE {fetch[(k, 'FETCH_SIZE')]:.1f} KiB, "
                   f"WRITE_SIZE {write.get((k, 'WRITE_SIZE'), 0.0):.1f} KiB raw per dispatch (median).")
    what = ("every copied block read once and written once" if copy else
            "KV of every context token once, shared blocks once, + Q" + (" + output" if p.query_start is not None else ""))
    out += ["", f"Per launch after scaling: {fetch_b / 1e6:.2f} MB read, {write_b / 1e6:.2f} MB written; algorithmic "
                f"bytes ({what}) {alg / 1e6:.2f} MB; measured / "
                f"algorithmic = {(fetch_b + write_b) / alg:.4f}.",
            "", f"Kernel sources hash {res['kernel_source_sha']} (comments and blank space removed); bench.py uses "
                f"these figures only while it matches."]
    print("\n".join(out))


def counters(args):
    merged, counts = {}, {}
    for d in args.dirs:
        m, n = counters_of(d)
        merged.update(m)
        counts.update(n)
    kernels = sorted({k for (k, c) in merged if is_main(k) or is_reduce(k)})
    names = sorted({c for (k, c) in merged})
    out = [f"# Counters: {args.config}", "", "Commands (repository root, one MI355X), one counter set per run:", "",
           "```"] + args.command + ["```", "", "Per dispatch (median over dispatches) of the attention kernel(s):", "",
                                    "| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
    for k in kernels:
        vals = []
        for c in names:
            v = merged.get((k, c))
            vals.append("" if v is None else (f"{v:.4g}" if abs(v) < 1e6 else f"{v:.4e}"))
        out.append(f"| `{short(k, 80)}` | " + " | ".join(vals) + " |")
    out += ["", "Definitions (rocprofv3's derived metrics on gfx950):", ""]
    for c in names:
        if c in EXPRESSIONS:
            out.append(f"- {c}: {EXPRESSIONS[c]}")
    hit, miss = None, None
    for k in kernels:
        if (k, "TCC_HIT_sum") in merged and (k, "TCC_MISS_sum") in merged:
            hit, miss = merged[(k, "TCC_HIT_sum")], merged[(k, "TCC_MISS_sum")]
            out.append(f"- L2 hit rate of `{short(k, 60)}`: {100 * hit / (hit + miss):.1f}% "
                       f"(TCC_HIT / (TCC_HIT + TCC_MISS))")
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("kind", choices=["trace", "traffic", "counters"])
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--config", required=True)
    ap.add_argument("--bench", help="the bench.py JSON line of the traced command")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--cold", type=int, default=0,
                    help="the last N attention launches are cold launches, where the bench JSON does not say")
    ap.add_argument("--json", help="traffic: where to write the JSON bench.py reads")
    ap.add_argument("--calibration", action="append", default=[],
                    help="traffic: counter folders of runs with bench.py --calibrate-copy, for the scale factors")
    args = ap.parse_args(argv)
    {"trace": trace, "traffic": traffic, "counters": counters}[args.kind](args)


if __name__ == "__main__":
    main()
