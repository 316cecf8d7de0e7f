"""bench.py's modes run end to end on the GPU and print one well-formed line.

Each mode runs bench.py as a child process on the tiny workload (2**20
parameters, 4 ranks): the default line with the CPU oracle's baseline, a
HIP-graph replay, cold caches, and the checkpoint benchmark.  The round of
GPU tests would otherwise never run these branches of bench.py.
"""

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TINY = ["--workload", "tiny_nd4_z2", "--steps", "3", "--warmup", "1"]


def _bench(*args, timeout=300):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"bench.py {' '.join(args)}", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                       text=True, timeout=timeout)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, p.stdout[-3000:]
    return json.loads(lines[0])


def _step_line(d):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["unit"] == "params/s" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "tiny_nd4_z2"
    rf = d["roofline"]
    assert {"bound", "achieved", "peak", "unit", "frac", "traffic"} <= set(rf)
    assert rf["achieved"] > 0 and rf["peak"] == 8000.0 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    sp = rf["achieved_per_step"]
    assert 0 < sp["min"] <= sp["median"] <= sp["max"] and sp["steps"] == d["steps"]
    assert d["step_flag"] == 0


def test_default_line_with_cpu_baseline():
    d = _bench(*TINY)
    _step_line(d)
    cb = d["cpu_baseline"]
    assert {"value", "unit", "cores", "kind", "sample", "gbs", "cpu"} <= set(cb)
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["gbs"] > 0
    assert d["sample_parity_reduced_bit_exact"] is True
    assert d["config"]["hip_graph"] is False and d["config"]["caches"] == "hot"


def test_graph_replay():
    d = _bench(*TINY, "--graph", "--no-cpu-baseline")
    _step_line(d)
    assert d["config"]["hip_graph"] is True and "cpu_baseline" not in d


def test_cold_caches():
    d = _bench(*TINY, "--flush-mb", "64", "--no-cpu-baseline")
    _step_line(d)
    assert d["config"]["caches"].startswith("64 MiB")


def test_checkpoint(tmp_path):
    d = _bench("--checkpoint", str(tmp_path), "--workload", "tiny_nd4_z2")
    assert d["unit"] == "GB/s" and d["restore_bit_exact"] is True
    assert d["save_gbs_median"] > 0 and d["restore_same_partition_gbs"] > 0 and d["restore_resharded_gbs"] > 0
    assert not any(p.name.startswith("zf-ckpt-") for p in tmp_path.iterdir())    # removed afterwards
