"""One rank's step driven from a plain C program, through the C ABI alone.

tests/c_step_driver.c allocates with hipMalloc and calls zero_reduce_shard,
zero_grad_norm and zero_adam_step; no Python binding and no PyTorch is
involved in the step.  Its outputs are checked like the binding's: the
reduced gradient bit for bit against the oracle, the norm and clip multiplier
within the bounds in tolerance.py, and AdamW within 1e-9 + 1e-6 relative (one
16-bit ulp) of the oracle and bit for bit when the clip multipliers agree.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import rounding, step
from oracle.step import AdamHparams
from tolerance import adam_parity, coef_ok, norm_ok

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "zero_sharded_mixed_flat_amd", "lib")
SOURCE = os.path.join(ROOT, "tests", "c_step_driver.c")
HIP = "/opt/rocm"
HP = AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)   # as in the C program
CODE = {"f16": 1, "bf16": 2}


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path_factory.mktemp("c_driver") / "c_step_driver"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    f"-I{HIP}/include", f"-I{INCLUDE}", SOURCE, "-o", str(exe), f"-L{LIBDIR}", "-lzero_flat",
                    f"-L{HIP}/lib", "-lamdhip64", f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{HIP}/lib"], check=True)
    return exe


@pytest.mark.parametrize("dtype, nd, n, std", [
    ("bf16", 8, 100_003, 1e-2),      # ragged tail; the norm is about 3, so clipping is active
    ("f16", 5, 70_001, 1e-3),        # Nd not a power of two: IEEE division by Nd
    ("bf16", 64, 4_099, 1e-4)])      # 64 contributions through the kernel-argument table
def test_c_program_step(driver, tmp_path, dtype, nd, n, std):
    print(f"C driver dtype={dtype} nd={nd} n={n}", flush=True)
    rng = np.random.default_rng(nd * 1_000_003 + n)
    contribs = [rounding.narrow((rng.standard_normal(n) * std).astype(np.float32), dtype) for _ in range(nd)]
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    np.concatenate(contribs).tofile(tmp_path / "contribs.bin")
    for name, a in (("master", master), ("m", m), ("v", v)):
        a.tofile(tmp_path / f"{name}.bin")

    p = subprocess.run([str(driver), str(tmp_path), str(n), str(nd), str(CODE[dtype])], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    reduced = np.fromfile(tmp_path / "out_reduced.bin", np.uint16)
    got = tuple(np.fromfile(tmp_path / f"out_{k}.bin", np.float32) for k in ("master", "m", "v")) + (
        np.fromfile(tmp_path / "out_param.bin", np.uint16),)
    raw = (tmp_path / "out_scalars.bin").read_bytes()
    norm = np.frombuffer(raw[:8], np.float64)[0]
    coef = np.frombuffer(raw[8:12], np.float32)[0]
    flag = np.frombuffer(raw[12:16], np.int32)[0]

    ref_reduced, bad = step.reduce_shard(contribs, dtype)
    assert not bad and flag == 0
    assert np.array_equal(reduced, ref_reduced)
    ref_norm = step.norm_from_sumsq(step.sumsq_exact(ref_reduced, dtype))
    norm_ok(norm, ref_norm, n)
    ref_coef = step.clip_coef(ref_norm, HP.max_norm)
    coef_ok(coef, ref_coef)
    if std == 1e-2:
        assert coef < 1.0
    ref = step.adam_update(master, m, v, ref_reduced, dtype, HP, 1, ref_coef, dtype)
    adam_parity(got, ref, dtype, "C driver", same=coef == ref_coef)
