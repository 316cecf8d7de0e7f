"""Whole-array GPU parity at full size for the single-rank ZeRO-1/2 layouts.

Every element of the rank's step is compared with the oracle: the reduced
gradient bit for bit, the exact norm of the whole reduced gradient (the sum of
the oracle's exact per-chunk sums of squares), and master, m, v and the
16-bit parameters within 1e-9 + 1e-6 relative and one 16-bit ulp, and bit for
bit whenever the device's clip multiplier equals the oracle's.  The inputs are the workload's
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
from tolerance import adam_parity, coef_ok, norm_ok
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
    norm_ok(run.norm.item(), norm, run.n)
    coef_ok(run.coef.item(), coef)
    assert float(coef) < 1.0                                  # clipping is active
    hp = AdamHparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                     inv_loss_scale=w.inv_loss_scale, max_norm=w.max_norm)
    dev_coef = np.float32(run.coef.item())

    def adam_chunk(c):
        lo, hi = c
        inputs = tuple(s[lo:hi] for s in state0)
        ref = step.adam_update(*inputs, reduced_ref[lo], w.grad_dtype, hp, 1, coef, w.param_dtype)
        got = tuple(s[lo:hi] for s in state_gpu) + (param_gpu[lo:hi],)
        adam_parity(got, ref, w.param_dtype, f"[{lo}, {hi})", same=dev_coef == coef)
        return hi - lo

    with ThreadPoolExecutor(THREADS) as ex:
        assert sum(ex.map(adam_chunk, chunks)) == n
    del run


def test_full_shard_zero3_and_gathered_layers(runner):
    # The 7.5e9-parameter, 64-rank ZeRO-3 workload: the rank's whole shard
    # (reduce over 64 ranks, exact norm, AdamW), then four whole layers of the
    # gathered buffer -- the other 63 owners' slices bit for bit, the rank's
    # own against the oracle's 16-bit parameters.
    from oracle import partition
    from tolerance import param16_ok
    w = workloads.get("paper_7p5b_nd64_z3")
    _note("full-shard paper_7p5b_nd64_z3: allocating")
    run = runner.RankStep(w, seed=13)
    n = run.n
    plan = partition.make_plan(w.units, w.nd, w.stage, w.align)
    contribs = [_host16(c) for c in run.contribs(0)]
    state0 = [t[0].cpu().numpy().copy() for t in (run.master, run.m, run.v)]
    layers = [0, 17, 30, len(plan.units) - 1]
    others = {u: [_host16(run.shards[r][plan.units[u].shard_base:plan.units[u].shard_base + plan.units[u].slice_numel])
                  for r in range(w.nd)] for u in layers}
    _note(f"full-shard: step over n={n}, oracle on {THREADS} threads")
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
        assert not bad and np.array_equal(reduced, reduced_gpu[lo:hi]), f"reduced gradient in [{lo}, {hi})"
        reduced_ref[lo] = reduced
        return step.sumsq_exact(reduced, w.grad_dtype, w.inv_loss_scale)

    with ThreadPoolExecutor(THREADS) as ex:
        norm = step.norm_from_sumsq(sum(ex.map(reduce_chunk, chunks)))
    del contribs
    coef = step.clip_coef(norm, w.max_norm)
    norm_ok(run.norm.item(), norm, run.n)
    coef_ok(run.coef.item(), coef)
    assert float(coef) < 1.0
    hp = AdamHparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                     inv_loss_scale=w.inv_loss_scale, max_norm=w.max_norm)
    dev_coef = np.float32(run.coef.item())
    bits_ref = np.empty(n, np.uint16)

    def adam_chunk(c):
        lo, hi = c
        inputs = tuple(s[lo:hi] for s in state0)
        ref = step.adam_update(*inputs, reduced_ref[lo], w.grad_dtype, hp, 1, coef, w.param_dtype)
        got = tuple(s[lo:hi] for s in state_gpu) + (param_gpu[lo:hi],)
        adam_parity(got, ref, w.param_dtype, f"[{lo}, {hi})", same=dev_coef == coef)
        bits_ref[lo:hi] = ref[3]
        return hi - lo

    with ThreadPoolExecutor(THREADS) as ex:
        assert sum(ex.map(adam_chunk, chunks)) == n
    for u in layers:
        unit = plan.units[u]
        for r in range(w.nd):
            dst = unit.full_base + r * unit.slice_numel
            got = _host16(run.full[dst:dst + unit.slice_numel])
            if r == w.rank:
                # the rank's own slice: its updated parameters, against the oracle's
                own = bits_ref[unit.shard_base:unit.shard_base + unit.slice_numel]
                param16_ok(got, own, w.param_dtype, f"layer {u} own slice")
                assert np.array_equal(got, param_gpu[unit.shard_base:unit.shard_base + unit.slice_numel])
            else:
                assert np.array_equal(got, others[u][r]), f"layer {u} owner {r}"
    del run


def test_sampled_chunks_owner_update_175b(runner):
    # The 175e9-parameter, 16-rank owner update (1.09e10 owned elements): the
    # exact norm of the whole tiled gradient, and 64 random 2^24-element chunks
    # plus the first and the last, element by element.
    w = workloads.get("gpt3_175b_nd16_z1")
    period = (1 << 20) + 37
    _note("sampled gpt3_175b_nd16_z1: allocating")
    run = runner.RankStep(w, seed=17, tile_period=period)
    n = run.n
    rng = np.random.default_rng(5)
    offs = sorted({0, n - CHUNK} | {int(x) for x in rng.integers(0, n - CHUNK, 64)})
    grads = {o: _host16(run.grad[o:o + CHUNK]) for o in offs}
    states = {o: tuple(t[0, o:o + CHUNK].cpu().numpy().copy() for t in (run.master, run.m, run.v)) for o in offs}
    period_grad = _host16(run.grad[:period])
    _note(f"sampled: step over n={n}, {len(offs)} chunks")
    run.step()
    torch.cuda.synchronize()
    assert int(run.flag.item()) == 0
    whole = step.sumsq_exact(period_grad, w.grad_dtype, w.inv_loss_scale)
    tail = step.sumsq_exact(period_grad[:n % period], w.grad_dtype, w.inv_loss_scale)
    norm = step.norm_from_sumsq((n // period) * whole + tail)
    coef = step.clip_coef(norm, w.max_norm)
    norm_ok(run.norm.item(), norm, run.n)
    coef_ok(run.coef.item(), coef)
    assert float(coef) < 1.0
    hp = AdamHparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                     inv_loss_scale=w.inv_loss_scale, max_norm=w.max_norm)
    dev_coef = np.float32(run.coef.item())
    got_all = {o: tuple(t[0, o:o + CHUNK].cpu().numpy() for t in (run.master, run.m, run.v))
               + (_host16(run.param_out(0)[o:o + CHUNK]),) for o in offs}

    def check(o):
        ref = step.adam_update(*states[o], grads[o], w.grad_dtype, hp, 1, coef, w.param_dtype)
        adam_parity(got_all[o], ref, w.param_dtype, f"@ {o}", same=dev_coef == coef)
        return CHUNK

    with ThreadPoolExecutor(THREADS) as ex:
        assert sum(ex.map(check, offs)) == CHUNK * len(offs)
    del run
