"""The device's fp32 -> 16-bit rounding, over every finite fp32 pattern.

With lr = 0, weight decay 0 and zero gradient, m and v, AdamW leaves the
master unchanged (p' = p - 0) and writes round_to_nearest_even_16(p) as the
parameter (CMU 11-868 Lecture 18 notes §2.2 step 4: the fp32 master is
copied to the 16-bit parameter).  All 2^32 - 2^24 finite fp32 patterns go
through zero_adam_step in 2^28-element chunks, for fp16 and bf16, and the
parameters are compared bit for bit with `oracle.rounding.narrow` (numpy's
float16 cast, and bf16 written out from its definition); the master must
come back unchanged.  Non-finite patterns (exponent all ones) are replaced
by zero on both sides.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import rounding

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28
PART = 1 << 24
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import abi as _abi
    return _abi


def _patterns_host(lo, hi):
    u = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32)
    u[(u & 0x7F800000) == 0x7F800000] = 0
    return u.view(np.float32)


def _expected(lo, dtype):
    out = np.empty(CHUNK, np.uint16)

    def part(k):
        a = lo + k * PART
        out[k * PART:(k + 1) * PART] = rounding.narrow(_patterns_host(a, a + PART), dtype)

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(part, range(CHUNK // PART)))
    return out


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_finite_fp32_pattern_rounds_like_the_oracle(abi, dtype):
    hp = abi.adam_hparams(0.0, 0.9, 0.999, 1e-8, 0.0, 1.0, 1)
    master = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    m = torch.zeros(CHUNK, dtype=torch.float32, device="cuda")
    v = torch.zeros(CHUNK, dtype=torch.float32, device="cuda")
    grad = torch.zeros(CHUNK, dtype=TORCH16[dtype], device="cuda")
    param = torch.empty(CHUNK, dtype=TORCH16[dtype], device="cuda")
    coef = torch.ones(1, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    exp_mask = torch.tensor(0x7F800000, dtype=torch.int32, device="cuda")
    for c in range(1 << 32 >> 28):
        lo = c * CHUNK
        print(f"rounding {dtype}: patterns [{lo:#010x}, {lo + CHUNK:#010x})", flush=True)
        bits = torch.arange(lo, lo + CHUNK, dtype=torch.int64, device="cuda").to(torch.int32)
        bits[(bits & exp_mask) == exp_mask] = 0
        master.view(torch.int32).copy_(bits)
        m.zero_()
        v.zero_()
        abi.zero_adam_step(master, m, v, grad, dtype, CHUNK, hp, coef, flag, param, dtype)
        expect = _expected(lo, dtype)              # on host threads while the GPU works
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        assert torch.equal(master.view(torch.int32), bits), "the master changed"
        got = param.view(torch.int16).cpu().numpy().view(np.uint16)
        bad = np.flatnonzero(got != expect)
        assert bad.size == 0, f"{bad.size} patterns differ, e.g. fp32 {_patterns_host(lo + int(bad[0]), lo + int(bad[0]) + 1)}" \
                              f" -> {got[bad[0]]:#06x}, oracle {expect[bad[0]]:#06x}"
        del bits
