"""Steps driven from plain C programs, through the C ABI alone.

tests/c_step_driver.c allocates with hipMalloc and calls zero_reduce_shard,
zero_grad_norm and zero_adam_step; no Python binding and no PyTorch is
involved in the step.  Its outputs are checked like the binding's: the
reduced gradient bit for bit against the oracle, the norm and clip multiplier
within the bounds in tolerance.py, and AdamW within 1e-9 + 1e-6 relative (one
16-bit ulp) of the oracle and bit for bit when the clip multipliers agree.

tests/c_graph_driver.c steps every rank of a group on one GPU with the
all-owner calls and the device step count, step 1 eagerly and steps 2 and 3
as launches of the step captured once in a HIP graph, with new gradients
copied in between; the result must be the oracle's three-step sequence.
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
GRAPH_SOURCE = os.path.join(ROOT, "tests", "c_graph_driver.c")
HIP = "/opt/rocm"
HP = AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)   # as in the C program
CODE = {"f16": 1, "bf16": 2}


def _compile(tmp_path_factory, source, name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path_factory.mktemp("c_driver") / name
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    f"-I{HIP}/include", f"-I{INCLUDE}", source, "-o", str(exe), f"-L{LIBDIR}", "-lzero_flat",
                    f"-L{HIP}/lib", "-lamdhip64", f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{HIP}/lib"], check=True)
    return exe


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    return _compile(tmp_path_factory, SOURCE, "c_step_driver")


@pytest.fixture(scope="module")
def graph_driver(tmp_path_factory):
    return _compile(tmp_path_factory, GRAPH_SOURCE, "c_graph_driver")


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


HP_GRAPH = AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_norm=1.0)  # as in the C program


@pytest.mark.parametrize("dtype, psi, nd, std", [("f16", 1 << 18, 4, 1e-3), ("bf16", 100_003, 8, 1e-2)])
def test_c_program_graph_replays(graph_driver, tmp_path, dtype, psi, nd, std):
    print(f"C graph driver dtype={dtype} psi={psi} nd={nd}", flush=True)
    from oracle import partition
    plan = partition.make_plan([psi], nd, 2, 8)
    rng = np.random.default_rng(psi + nd)
    grads = [[rounding.narrow((rng.standard_normal(psi) * std).astype(np.float32), dtype) for _ in range(nd)]
             for _ in range(3)]
    full = [(rng.standard_normal(psi) * s).astype(np.float32) for s in (0.02, 1e-4)]
    full.append(np.abs(rng.standard_normal(psi) * 1e-6).astype(np.float32))
    states = [tuple(partition.shard_of(plan, a, o) for a in full) for o in range(nd)]
    np.concatenate([g for step_grads in grads for g in step_grads]).tofile(tmp_path / "grads.bin")
    for k, name in enumerate(("master", "m", "v")):
        np.concatenate([st[k] for st in states]).tofile(tmp_path / f"{name}.bin")

    p = subprocess.run([str(graph_driver), str(tmp_path), str(psi), str(nd), str(CODE[dtype])], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    ref = step.step_sequence(plan, grads, states, HP_GRAPH, dtype, dtype)
    assert [r["t"] for r in ref] == [1, 2, 3] and not any(r["skipped"] for r in ref)
    got = tuple(np.fromfile(tmp_path / f"out_{k}.bin", np.float32) for k in ("master", "m", "v"))
    n = plan.shard_numel
    param = np.fromfile(tmp_path / "out_param.bin", np.uint16)
    for o in range(nd):
        mine = tuple(a[o * n:(o + 1) * n] for a in got) + (param[o * n:(o + 1) * n],)
        expect = tuple(ref[2]["states"][o]) + (ref[2]["full"][o * n:(o + 1) * n],)
        adam_parity(mine, expect, dtype, f"owner {o} after the second replay")
    state = np.fromfile(tmp_path / "out_state.bin", np.int64)
    assert tuple(state[:3]) == (4, 3, 0)                         # t, applied, skipped
