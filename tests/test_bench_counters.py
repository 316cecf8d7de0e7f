"""bench.py's HBM-traffic bookkeeping, on the CPU.

rocprofv3's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what
the same counters read for the reference copy of known size; each phase
kernel's scaled bytes go into profiles/traffic.json under a hash of the
kernel's sources, and bench.py reports them only while that hash holds.
Synthetic counter files stand in for rocprofv3's here.
"""

import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

ADAM = "void zf::(anonymous namespace)::adam_kernel<2, 2, false>(float*)"
GATHER = "void zf::(anonymous namespace)::gather_kernel<false>(zf::Ptrs64)"
COPY_GRID = bench.COPY_ELEMS // 8 // 2
PHASES = {"adam": {"kernel": "adam_kernel", "bytes_per_launch": 28.0e9, "launches": 1},
          "gather": {"kernel": "gather_kernel", "bytes_per_launch": 6.25e8, "launches": 48}}


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for name, grid, value in rows:
            w.writerow([name, grid, counter, value])
            w.writerow([name, grid, "OTHER_COUNTER", 1.0])          # ignored


def _files(tmp_path, copy_fetch_kib, copy_write_kib):
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counters(fetch, "FETCH_SIZE", [(GATHER, COPY_GRID, copy_fetch_kib), (ADAM, 1024, 7.0e6), (ADAM, 1024, 7.2e6),
                                    (GATHER, 4096, 1.6e5), ("at::native::fill", 8, 5.0)])
    _counters(write, "WRITE_SIZE", [(GATHER, COPY_GRID, copy_write_kib), (ADAM, 1024, 1.4e7), (ADAM, 1024, 1.4e7),
                                    (GATHER, 4096, 3.0e5)])
    return str(fetch), str(write)


def test_scaled_bytes_per_kernel(tmp_path):
    ref_kib = bench.COPY_BYTES_EACH_WAY / 1024
    text, entry = bench.summarize_counters(*_files(tmp_path, ref_kib / 2, ref_kib), PHASES, ["cmd fetch", "cmd write"])
    assert entry["fetch_scale"] == pytest.approx(2.0) and entry["write_scale"] == pytest.approx(1.0)
    adam = entry["kernels"]["adam_kernel"]
    assert adam["bytes_read"] == pytest.approx(7.1e6 * 1024 * 2)        # mean of the two dispatches, scaled
    assert adam["bytes_written"] == pytest.approx(1.4e7 * 1024)
    assert adam["bytes_per_launch"] == pytest.approx(adam["bytes_read"] + adam["bytes_written"])
    assert adam["algorithmic_bytes_per_launch"] == 28.0e9
    assert adam["kernel_source_sha256_16"] == bench.kernel_source_hash("adam_kernel")
    # the reference copy is not taken for the gather phase; the per-layer dispatch is
    assert entry["kernels"]["gather_kernel"]["grid"] == 4096
    assert entry["kernels"]["gather_kernel"]["bytes_per_launch"] == pytest.approx(1.6e5 * 1024 * 2 + 3.0e5 * 1024)
    ratio = (7.1e6 * 1024 * 2 + 1.4e7 * 1024) / 28.0e9
    assert f"{ratio:.4f}x" in text and "cmd fetch" in text and "cmd write" in text
    assert "fill" not in text                                            # not this library's kernel


def test_no_reference_copy_is_an_error(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counters(fetch, "FETCH_SIZE", [(ADAM, 1024, 7.0e6)])
    _counters(write, "WRITE_SIZE", [(ADAM, 1024, 1.4e7)])
    with pytest.raises(RuntimeError, match="reference copy"):
        bench.summarize_counters(str(fetch), str(write), PHASES, [])


def test_traffic_is_used_only_while_the_sources_hash_the_same(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("w", "adam_kernel") is None                   # no file
    good = {"kernel_source_sha256_16": bench.kernel_source_hash("adam_kernel"), "bytes_per_launch": 2.81e10}
    stale = dict(good, kernel_source_sha256_16="0" * 16)
    path.write_text(json.dumps({"w": {"kernels": {"adam_kernel": good, "reduce_kernel": stale}}}))
    assert bench.measured_traffic("w", "adam_kernel") == 2.81e10
    assert bench.measured_traffic("w", "reduce_kernel") is None                 # sources changed since
    assert bench.measured_traffic("other", "adam_kernel") is None
    path.write_text("not json")
    assert bench.measured_traffic("w", "adam_kernel") is None


def test_source_hash_follows_the_kernel_file():
    kernels = {bench.kernel_source_hash(k) for k in ("adam_kernel", "reduce_kernel", "gather_kernel")}
    quant = {bench.kernel_source_hash(k) for k in ("quantize_span_kernel", "gather_dequant_kernel",
                                                  "dequantize_kernel")}
    assert len(kernels) == 1 and len(quant) == 1 and kernels != quant

