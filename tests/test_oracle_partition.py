"""Pins for oracle.partition: the pages' worked example, brute-force coverage,
and the shard sizes of the layouts the parity tests and the benchmark use."""

import os
import random

import numpy as np
import pytest

from oracle import partition
from zero_sharded_mixed_flat_amd import workloads


def test_printed_flat_partitions():
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_flat_partition.csv")
    with open(path) as f:
        rows = [line.strip().split(",") for line in f if line.strip() and not line.startswith("#")]
    assert rows
    for sizes, nd, per_rank, source in rows:
        sizes = [int(x) for x in sizes.split()]
        plan = partition.make_plan(sizes, nd=int(nd), stage=1, align=1)
        assert [plan.real_numel(r) for r in range(int(nd))] == [int(x) for x in per_rank.split()], source


def test_exercise6_flat_partition():
    # CMU 11-868 Lecture 18 notes §8 exercise 6 answer: tensors of 100, 60 and
    # 40 elements on 2 ranks; the flat partition gives each rank 100 elements,
    # rank 0 all of the first tensor, rank 1 the other two.
    plan = partition.make_plan([100, 60, 40], nd=2, stage=1, align=1)
    assert plan.shard_numel == 100
    assert [plan.real_numel(r) for r in range(2)] == [100, 100]
    assert partition.segments(plan, [100, 60, 40], 0) == [(0, 0, 0, 100)]
    assert partition.segments(plan, [100, 60, 40], 1) == [(1, 0, 0, 60), (2, 0, 60, 40)]


def test_exercise6_variant_tensor_straddles_ranks():
    # The exercise's second set of sizes (100, 30, 20), where the page works out
    # only the greedy per-tensor split.  The flat split is 75/75 and, as the
    # notes say of the flat scheme (§3.2), a tensor is cut across two ranks.
    plan = partition.make_plan([100, 30, 20], nd=2, stage=2, align=1)
    assert [plan.real_numel(r) for r in range(2)] == [75, 75]
    assert partition.segments(plan, [100, 30, 20], 0) == [(0, 0, 0, 75)]
    assert partition.segments(plan, [100, 30, 20], 1) == [(0, 75, 0, 25), (1, 0, 25, 30), (2, 0, 55, 20)]


def _brute_force_owner_map(units, nd, stage, align):
    """Independent enumeration: for every real element, who owns it and where."""
    owners = 1 if stage == 0 else nd
    flat_units = units if stage == 3 else [sum(units)]
    where = {}
    shard_pos = [0] * owners
    for ui, numel in enumerate(flat_units):
        per = -(-numel // owners)
        s = -(-per // align) * align
        for r in range(owners):
            for j in range(s):
                pos = r * s + j
                if pos < numel:
                    where.setdefault((ui, pos), []).append((r, shard_pos[r] + j))
            shard_pos[r] += s
    return where, flat_units


@pytest.mark.parametrize("seed", range(40))
def test_every_real_element_owned_exactly_once(seed):
    rng = random.Random(seed)
    n_units = rng.randint(1, 6)
    units = [rng.choice([0, 1, 7, rng.randint(1, 300)]) for _ in range(n_units)]
    if sum(units) == 0:
        units[0] = 5
    nd = rng.choice([1, 2, 3, 4, 5, 8, 16, 33])
    stage = rng.choice([0, 1, 2, 3])
    align = rng.choice([1, 2, 8])
    plan = partition.make_plan(units, nd, stage, align)
    where, flat_units = _brute_force_owner_map(units, nd, stage, align)
    assert all(len(v) == 1 for v in where.values())
    assert len(where) == sum(flat_units)
    # The plan's owned ranges and shard offsets agree with the enumeration.
    for ui, u in enumerate(plan.units):
        for r in range(plan.owners):
            lo, hi = plan.owned(r, ui)
            for pos in range(lo, hi):
                assert where[(ui, pos)] == [(r, u.shard_base + pos - r * u.slice_numel)]
    # Balance: nobody owns more than ceil(U/owners) + align - 1 of a unit.
    for ui, u in enumerate(plan.units):
        for r in range(plan.owners):
            lo, hi = plan.owned(r, ui)
            assert hi - lo <= -(-u.numel // plan.owners) + align - 1
    # Padded sizes: padding per unit is < owners * align.
    for u in plan.units:
        assert 0 <= plan.owners * u.slice_numel - u.numel < plan.owners * align


@pytest.mark.parametrize("seed", range(10))
def test_shard_of_and_gather_invert_each_other(seed):
    rng = np.random.default_rng(seed)
    units = [int(x) for x in rng.integers(1, 200, size=rng.integers(1, 5))]
    nd = int(rng.choice([1, 2, 3, 4, 7]))
    stage = int(rng.choice([1, 2, 3]))
    plan = partition.make_plan(units, nd, stage, align=int(rng.choice([1, 8])))
    full = rng.integers(1, 60000, size=plan.psi).astype(np.uint16)
    shards = [partition.shard_of(plan, full, r) for r in range(plan.owners)]
    from oracle.step import gather
    padded = gather(plan, shards, np.zeros(plan.full_numel, np.uint16))
    assert np.array_equal(partition.unpad(plan, padded), full)


def test_layout_shard_sizes():
    # Derived shard sizes of the layouts used by the parity tests and bench:
    # 8.03e9 flat over 8 ranks; 7.5e9 as 48 layer units over 64 ranks; the
    # GPT-2 1.5B layout over 16 ranks; 175e9 over 16 ranks.
    expect = {
        "llama3_8b_nd8_z2": 1_003_750_000,
        "paper_7p5b_nd64_z3": 117_187_584,
        "gpt2_1p5b_nd16_z1": 97_350_704,
        "gpt3_175b_nd16_z1": 10_937_500_000,
    }
    for name, shard in expect.items():
        w = workloads.get(name)
        plan = partition.make_plan(w.units, w.nd, w.stage, w.align)
        assert plan.shard_numel == shard, name
    w = workloads.get("paper_7p5b_nd64_z3")
    plan = partition.make_plan(w.units, w.nd, w.stage, w.align)
    assert plan.units[0].slice_numel == 2_441_408
    assert plan.full_numel == 7_500_005_376


def test_gpt2_layout_ragged_cut():
    # GPT-2 1.5B as laid out by the tensor list (48 layers, h = 1600, 4h MLP,
    # vocab 50257): 580 tensors, 1,557,611,200 parameters.  The flat split over
    # 16 ranks cuts tensors in the middle; rank 5's pieces cover its shard.
    w = workloads.get("gpt2_1p5b_nd16_z1")
    assert len(w.tensors) == 580
    assert sum(w.tensors) == 1_557_611_200
    plan = partition.make_plan(w.units, w.nd, w.stage, w.align)
    total = 0
    for r in range(w.nd):
        segs = partition.segments(plan, w.tensors, r)
        covered = sum(s[3] for s in segs)
        assert covered == plan.real_numel(r)
        offs = [s[2] for s in segs]
        assert offs == sorted(offs)
        total += covered
    assert total == plan.psi
    segs5 = partition.segments(plan, w.tensors, 5)
    first, last = segs5[0], segs5[-1]
    assert first[1] > 0 or last[1] + last[3] < w.tensors[last[0]]   # a tensor is cut
    assert plan.real_numel(15) == plan.shard_numel - 64


def test_invalid_arguments():
    with pytest.raises(ValueError):
        partition.make_plan([10], nd=0, stage=1)
    with pytest.raises(ValueError):
        partition.make_plan([10], nd=2, stage=4)
    with pytest.raises(ValueError):
        partition.make_plan([], nd=2, stage=1)
    with pytest.raises(ValueError):
        partition.make_plan([10], nd=2, stage=1, align=0)
