"""Whole-array GPU parity at full size for the single-rank ZeRO-1/2 layouts.

Every element of the rank's step is compared with the oracle: the reduced
gradient bit for bit, the exact norm of the whole reduced gradient (the sum of
the oracle's exact per-chunk sums of squares), and master, m, v and the
16-bit parameters to the derived tolerance.  The inputs are the workload's
own seeded draws (no tiling), copied to the host before the step; the oracle
runs chunk by chunk on host threads (numpy releases the interpreter lock in
its array operations).
"""

import gc
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import step
from oracle.step import AdamHparams
from tolerance import adam_ok
from zero_sharded_mixed_flat_amd import synth, workloads

pytestmark = pytest.mark.gpu

CHUNK = 1 << 24
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture
def runner():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import runner as _runner
    yield _runner
    gc.collect()
    torch.cuda.empty_cache()


def _note(msg):
    print(msg, flush=True)


def _host16(t):
    return synth.bits(t)


@pytest.mark.parametrize("name", ["gpt2_1p5b_nd16_z1", "llama3_8b_nd8_z2"])
def test_full_array_step(runner, name):
    w = workloads.get(name)
    _note(f"full-array {name}: allocating")
    run = runner.RankStep(w, seed=9)
    n = run.n
    contribs = [_host16(c) for c in run.contribs(0)]
    state0 = [t[0].cpu().numpy().copy() for t in (run.master, run.m, run.v)]
    _note(f"full-array {name}: step over n={n}, oracle on {THREADS} threads")
    run.step()
    torch.cuda.synchronize()
    assert int(run.flag.item()) == 0
    reduced_gpu = _host16(run.reduced[0])
    state_gpu = [t[0].cpu().numpy() for t in (run.master, run.m, run.v)]
    param_gpu = _host16(run.param_out(0))
    chunks = [(lo, min(n, lo + CHUNK)) for lo in range(0, n, CHUNK)]

    reduced_ref = {}

    def reduce_chunk(c):
        lo, hi = c
        reduced, bad = step.reduce_shard([x[lo:hi] for x in contribs], w.grad_dtype)
        assert not bad
        assert np.array_equal(reduced, reduced_gpu[lo:hi]), f"reduced gradient differs in [{lo}, {hi})"
        reduced_ref[lo] = reduced
        return step.sumsq_exact(reduced, w.grad_dtype, w.inv_loss_scale)

    with ThreadPoolExecutor(THREADS) as ex:
        sumsq = sum(ex.map(reduce_chunk, chunks))
    del contribs
    norm = step.norm_from_sumsq(sumsq)
    coef = step.clip_coef(norm, w.max_norm)
    _note(f"  norm gpu {run.norm.item():.12g} oracle {norm:.12g}, coef {float(coef):.8g}")
    assert run.norm.item() == pytest.approx(norm, rel=1e-5)
    assert float(coef) < 1.0                                  # clipping is active
    hp = AdamHparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                     inv_loss_scale=w.inv_loss_scale, max_norm=w.max_norm)

    def adam_chunk(c):
        lo, hi = c
        inputs = tuple(s[lo:hi] for s in state0)
        ref = step.adam_update(*inputs, reduced_ref[lo], w.grad_dtype, hp, 1, coef, w.param_dtype)
        got = tuple(s[lo:hi] for s in state_gpu) + (param_gpu[lo:hi],)
        adam_ok(got, ref, inputs, reduced_ref[lo], w.grad_dtype, hp, 1, coef, w.param_dtype, f"[{lo}, {hi})")
        return hi - lo

    with ThreadPoolExecutor(THREADS) as ex:
        assert sum(ex.map(adam_chunk, chunks)) == n
    del run
