"""Pins for the oracle's resharding (restoring sharded state under another partition).

026 notes §五: restoring at a different degree of parallelism must re-own the
state, keeping the parameter order and the moment belonging to each
parameter; a single step after the restore is compared with an uninterrupted
run, and the device count is changed.

Pages cited by short name:
  026 notes  "026｜ZeRO：数据并行中，没必要让每张卡保存全部训练状态" (wq-win.github.io)
"""

import numpy as np
import pytest

from oracle import partition, rounding, step
from oracle.step import AdamHparams


def _random_plan(rng, psi=None):
    n_units = int(rng.integers(1, 5))
    units = [int(x) for x in rng.integers(0, 3000, n_units)]
    if psi is not None:
        units[-1] += psi - sum(units)
        if units[-1] < 0:
            units = [psi]
    nd = int(rng.integers(1, 20))
    stage = int(rng.integers(0, 4))
    align = int(rng.choice([1, 8, 256]))
    return partition.make_plan(units, nd, stage, align)


def _shards(plan, v):
    return [partition.shard_of(plan, v, r) for r in range(plan.owners)]


@pytest.mark.parametrize("seed", range(12))
def test_merge_inverts_shard_of(seed):
    rng = np.random.default_rng(seed)
    plan = _random_plan(rng)
    v = rng.standard_normal(plan.psi).astype(np.float32)
    assert np.array_equal(partition.merge(plan, _shards(plan, v)), v)


@pytest.mark.parametrize("seed", range(12))
def test_reshard_between_random_plans(seed):
    rng = np.random.default_rng(100 + seed)
    old = _random_plan(rng)
    new = _random_plan(rng, psi=old.psi)
    assert new.psi == old.psi
    # label every parameter by its flat index: the new shard must hold the
    # labels of exactly the flat positions the new plan gives it, in order
    labels = np.arange(old.psi, dtype=np.int64) + 1
    old_shards = _shards(old, labels)
    for r in range(new.owners):
        got = partition.reshard(old, old_shards, new, r)
        flat_base, expect = 0, np.zeros(new.shard_numel, np.int64)
        for i, u in enumerate(new.units):
            lo, hi = new.owned(r, i)
            rr = 0 if new.owners == 1 else r
            expect[u.shard_base + lo - rr * u.slice_numel:u.shard_base + hi - rr * u.slice_numel] = \
                np.arange(flat_base + lo, flat_base + hi) + 1
            flat_base += u.numel
        assert np.array_equal(got, expect)
        # the runs move exactly the same elements; everything else is padding (zero)
        applied = np.zeros(new.shard_numel, np.int64)
        covered = np.zeros(new.shard_numel, bool)
        for orank, ooff, noff, ln in partition.reshard_segments(old, new, r):
            assert ln > 0 and not covered[noff:noff + ln].any()
            applied[noff:noff + ln] = old_shards[orank][ooff:ooff + ln]
            covered[noff:noff + ln] = True
        assert np.array_equal(applied, got) and np.array_equal(covered, got != 0)


def test_round_trip_8_16_8():
    rng = np.random.default_rng(7)
    units = [10_007, 33, 4096]
    p8 = partition.make_plan(units, 8, 3, 8)
    p16 = partition.make_plan(units, 16, 3, 8)
    v = rng.standard_normal(p8.psi).astype(np.float32)
    s8 = _shards(p8, v)
    s16 = [partition.reshard(p8, s8, p16, r) for r in range(16)]
    back = [partition.reshard(p16, s16, p8, r) for r in range(8)]
    for a, b in zip(back, s8):
        assert np.array_equal(a, b)


def test_stage_change_keeps_parameter_order():
    # ZeRO-2 (one flat unit) -> ZeRO-3 (one unit per layer) and back.
    rng = np.random.default_rng(3)
    layers = [5000, 5000, 123, 7777]
    z2 = partition.make_plan(layers, 4, 2, 8)
    z3 = partition.make_plan(layers, 6, 3, 256)
    v = rng.standard_normal(z2.psi).astype(np.float32)
    s3 = [partition.reshard(z2, _shards(z2, v), z3, r) for r in range(6)]
    assert np.array_equal(partition.merge(z3, s3), v)
    # a per-layer view: layer 2's parameters are where the flat order puts them
    assert np.array_equal(partition.merge(z3, s3)[10_000:10_123], v[10_000:10_123])


def test_same_plan_is_identity_and_psi_must_match():
    plan = partition.make_plan([1000], 3, 1, 8)
    v = np.arange(1000, dtype=np.float32)
    s = _shards(plan, v)
    for r in range(3):
        assert np.array_equal(partition.reshard(plan, s, plan, r), s[r])
    with pytest.raises(ValueError):
        partition.reshard(plan, s, partition.make_plan([1001], 3, 1, 8), 0)
    with pytest.raises(ValueError):
        partition.merge(plan, s[:2])


def test_step_after_reshard_equals_uninterrupted():
    # Two steps at Nd = 4, or one at Nd = 4, a restore at Nd = 8 and the second
    # there: the same parameters, m and v bit for bit.  Every rank sees the
    # same local gradient, so the data-parallel mean is that gradient at any Nd.
    rng = np.random.default_rng(11)
    units = [3001, 4096, 777]
    hp = AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    pa = partition.make_plan(units, 4, 3, 8)
    pb = partition.make_plan(units, 8, 2, 16)
    psi = pa.psi
    flat = [rng.standard_normal(psi).astype(np.float32) * s for s in (0.02, 1e-4, 1e-6)]
    flat[2] = np.abs(flat[2])
    grads = [rounding.narrow((rng.standard_normal(psi) * 1e-3).astype(np.float32), "f16") for _ in range(2)]

    def states_of(plan, vectors):
        return [tuple(partition.shard_of(plan, x, r) for x in vectors) for r in range(plan.owners)]

    def run(plan, states, g, t):
        out = step.step_sharded(plan, [g] * plan.nd, states, hp, t, "f16", "f16")
        assert not out["skipped"]
        return out["states"], out["full"]

    sa, _ = run(pa, states_of(pa, flat), grads[0], 1)
    sa2, full_a = run(pa, sa, grads[1], 2)
    merged_a = [partition.merge(pa, [s[k] for s in sa]) for k in range(3)]
    sb = [tuple(partition.reshard(pa, [s[k] for s in sa], pb, r) for k in range(3)) for r in range(8)]
    sb2, full_b = run(pb, sb, grads[1], 2)
    for k in range(3):
        assert np.array_equal(partition.merge(pa, [s[k] for s in sa2]), partition.merge(pb, [s[k] for s in sb2]))
    assert np.array_equal(partition.unpad(pa, full_a), partition.unpad(pb, full_b))
    assert not np.array_equal(merged_a[0], partition.merge(pa, [s[0] for s in sa2]))   # the step did move


def test_runs_break_at_padding_of_the_new_shard():
    # Rank 0 of the new plan holds all of a short layer, then padding, then
    # the start of the next layer; in the old flat plan those parameters are
    # contiguous, so only the new shard's gap splits the run.
    old = partition.make_plan([100, 5000], 2, 2, 8)
    new = partition.make_plan([100, 5000], 4, 3, 256)
    runs = partition.reshard_segments(old, new, 0)
    assert runs[:2] == [(0, 0, 0, 100), (0, 100, 256, 1280)]
    labels = np.arange(old.psi) + 1
    got = partition.reshard(old, _shards(old, labels), new, 0)
    assert np.all(got[100:256] == 0) and got[256] == 101
