"""rocprof_summary.py's kernel-trace summary splits bench.py's launches right (CPU).

bench.py runs, in order: settle steps, warm-up steps, the timed passes, then
the cold launches (each after a 512 MiB read).  The summary's warm figure must
average only the launches between the first two groups and the cold ones, and
its cold figure only the cold ones, taking the counts from the bench JSON line
whatever --cold says (a summary once averaged the cold launches in with the
warm ones when --cold 0 was passed).
"""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = "void pa::(anonymous namespace)::prefill_kernel<128>(pa::PrefillParams)"


def write_trace(d, durations_us):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 1_000_000
        for us in durations_us:
            w.writerow([KERNEL, t, t + int(round(us * 1000))])
            t += int(round(us * 1000)) + 5000
    with open(os.path.join(d, "run_kernel_stats.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        n = len(durations_us)
        w.writerow([KERNEL, n, sum(durations_us) / n * 1000, min(durations_us) * 1000, max(durations_us) * 1000, 100.0])


@pytest.mark.parametrize("cold_arg", ["0", "8"])
def test_warm_and_cold_launches_from_the_bench_json(tmp_path, cold_arg):
    settle, warmup, warm, cold = 40, 10, 30, 72
    durations = [300.0] * settle + [250.0] * warmup + [166.0] * warm + [190.0] * cold
    d = str(tmp_path / "kt")
    write_trace(d, durations)
    bench = {"settle_steps": settle, "warmup": warmup, "ms_per_step": 0.17, "value": 1.0, "unit": "tokens/s",
             "breakdown_us": {"cold_launches": cold},
             "roofline": {"unit": "TFLOP/s", "avg_launch_us": 166.0, "achieved": 777.0, "frac": 0.31,
                          "algorithmic_flops_per_launch": 1.289e11}}
    bj = str(tmp_path / "bench.json")
    with open(bj, "w") as f:
        json.dump(bench, f)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "rocprof_summary.py"), "trace", d, "--config",
                          "chunked-prefill", "--bench", bj, "--cold", cold_arg],
                         capture_output=True, text=True, check=True, cwd=ROOT).stdout
    assert f"{warm} warm launches: average 166.00 us" in out, out
    assert f"The last {cold} launches are bench.py's cold launches" in out and "average 190.00 us" in out, out
    assert "/ 166.00 us" in out, out  # the trace-based rate uses the warm average
