"""The largest sizes one call accepts: 2^34 elements (ZERO_MAX_ELEMS).

At that size the reduce's grid holds 2^23 blocks of 2^8 threads, the
partial sums fill 2^23 slots (the whole static scratch of the allocation-
free norm) and every index passes 2^32.  The reduce runs over 2 ranks in
place over rank 0's contribution (64 GiB of 16-bit data); sampled chunks
at the start, across the 2^31 and 2^32 element marks and at the end are
compared bit for bit with the oracle.  Both norm entry points (workspace
and static scratch) then take the norm of the 2^34-element reduced
gradient; each contribution is tiled with a ragged period, so the exact
sum of squares follows from one period (the tiling property the other
full-size tests use).  A size one past the limit is rejected.
"""

import numpy as np
import pytest
import torch

from oracle import rounding, step
from tolerance import coef_ok, norm_ok

pytestmark = pytest.mark.gpu

N = 1 << 34
PERIOD = (1 << 20) + 37
CHUNK = 1 << 20


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import abi as _abi
    return _abi


def _note(msg):
    print(msg, flush=True)


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _tiled(seed, std):
    rng = np.random.default_rng(seed)
    period = rounding.narrow((rng.standard_normal(PERIOD) * std).astype(np.float32), "bf16")
    t = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    t[:PERIOD].copy_(torch.from_numpy(period.view(np.int16)).view(torch.bfloat16))
    done = PERIOD
    while done < N:                      # doubling copies: the whole tensor repeats the period
        k = min(done, N - done)
        t[done:done + k].copy_(t[:k])
        done += k
    return t, period


def test_reduce_and_norms_at_the_element_limit(abi):
    _note(f"max size: two bf16 contributions of {N} elements (tiled, period {PERIOD})")
    a, pa = _tiled(1, 1e-4)
    b, pb = _tiled(2, 1e-4)
    offs = [0, (1 << 31) - CHUNK // 2, (1 << 32) - CHUNK // 2, N - CHUNK]
    inputs = {o: (_bits(a[o:o + CHUNK]), _bits(b[o:o + CHUNK])) for o in offs}
    ws = torch.empty(abi.zero_workspace_bytes(N, 1), dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    _note("max size: reduce in place over rank 0's contribution")
    abi.zero_reduce_shard([a, b], N, "bf16", 1.0, a, ws, 0, flag)
    norms = []
    for noalloc in (False, True):
        norm = torch.zeros(1, dtype=torch.float64, device="cuda")
        coef = torch.zeros(1, dtype=torch.float32, device="cuda")
        if noalloc:
            abi.zero_grad_norm_noalloc(a, N, "bf16", 1.0, None, 0, 1.0, flag, norm, coef)
        else:
            abi.zero_grad_norm(a, N, "bf16", 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
        torch.cuda.synchronize()
        norms.append((norm.item(), coef.item()))
    assert int(flag.item()) == 0
    for o in offs:
        ref, bad = step.reduce_shard(list(inputs[o]), "bf16")
        assert not bad and np.array_equal(_bits(a[o:o + CHUNK]), ref), f"reduced gradient at {o}"
    red_period, bad = step.reduce_shard([pa, pb], "bf16")
    assert not bad
    whole = step.sumsq_exact(red_period, "bf16")
    tail = step.sumsq_exact(red_period[:N % PERIOD], "bf16")
    ref_norm = step.norm_from_sumsq((N // PERIOD) * whole + tail)
    _note(f"max size: norms {norms}, oracle {ref_norm!r}")
    assert norms[0] == norms[1]                    # same kernels, same tree
    norm_ok(norms[0][0], ref_norm, N)
    coef_ok(norms[0][1], step.clip_coef(ref_norm, 1.0))
    del a, b, ws


def test_one_past_the_limit_is_rejected(abi):
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_reduce_shard([t.data_ptr(), t.data_ptr() + 2], N + 1, "bf16", 1.0, ws.data_ptr() + 64, ws, 0, flag,
                              workspace_bytes=1 << 40)
    assert e.value.code == abi.ZERO_EINVAL and "2^34" in str(e.value)
