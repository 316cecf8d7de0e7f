"""bench.py's host-side paths: the one-GPU refusal and the trace summary.

The summary is fed small rocprofv3-shaped CSV files and a bench result line
written here, so its grouping by grid size and its same-process comparison of
bench.py's HIP-event time with rocprofv3's average are checked without a GPU.
"""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

ADAM = "void zf::(anonymous namespace)::adam_kernel<2, 2, false>(float*, float*)"
RED = "void zf::(anonymous namespace)::reduce_kernel<2, 8>(zf::Ptrs64)"


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and p.stdout == ""
    assert "one GPU" in p.stderr and "--gpus 2" in p.stderr


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_with_bench_line(tmp_path):
    stats = tmp_path / "trace_kernel_stats.csv"
    _write(stats, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [[ADAM, 2, 5.0e6, 4.9e6, 5.1e6, 60.0], [RED, 2, 3.0e6, 2.9e6, 3.1e6, 36.0],
            ["at::native::fill_kernel", 3, 1e3, 1e3, 1e3, 0.1]])
    trace = tmp_path / "trace_kernel_trace.csv"
    rows = []
    for name, grid, dur in ((ADAM, 1024, 4.9e6), (ADAM, 1024, 5.1e6), (ADAM, 64, 1e4), (RED, 2048, 3.0e6)):
        rows.append([name, grid, 1, 1000, 1000 + int(dur)])
    _write(trace, ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Start_Timestamp", "End_Timestamp"], rows)
    log = tmp_path / "bench.log"
    line = {"metric": "m", "value": 1.0e11, "unit": "params/s", "ms_per_step": 8.2, "steps": 20, "warmup": 3,
            "roofline": {"kernel": "adam_kernel", "launch_ms": 5.05, "launches_per_step": 1, "achieved": 5600.0,
                         "unit": "GB/s", "peak": 8000.0, "frac": 0.7}}
    log.write_text("rocprofv3 noise\n" + json.dumps(line) + "\n")
    out = bench.summarize_trace(str(stats), "the command", str(log))
    assert "the command" in out
    assert "| `adam_kernel<2, 2, false>` | 1024 | 2 | 5000.0 | 4900.0 | 5100.0 |" in out
    assert "| `adam_kernel<2, 2, false>` | 64 | 1 | 10.0 |" in out
    # bench.py's 5050 us against the busiest adam group's 5000 us average
    assert "5050.0 us per launch" in out and "5000.0 us average" in out and "ratio 1.010" in out


def test_trace_summary_without_a_gpu_dispatch_for_the_roofline_kernel(tmp_path):
    stats = tmp_path / "trace_kernel_stats.csv"
    _write(stats, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"], [[RED, 1, 1e6, 1e6, 1e6, 99.0]])
    trace = tmp_path / "trace_kernel_trace.csv"
    _write(trace, ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Start_Timestamp", "End_Timestamp"],
           [[RED, 2048, 1, 0, 1000000]])
    log = tmp_path / "bench.log"
    log.write_text(json.dumps({"metric": "m", "value": 1.0, "unit": "params/s", "ms_per_step": 100.0, "steps": 2,
                               "warmup": 1, "roofline": {"kernel": "host_adam", "launch_ms": 90.0,
                                                         "launches_per_step": 1}}) + "\n")
    out = bench.summarize_trace(str(stats), "cmd", str(log))
    assert "runs no GPU dispatch to compare" in out
