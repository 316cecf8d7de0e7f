"""Resharding runs and sharded checkpoints on the host (no GPU needed).

The library's runs (``zero_plan_reshard``) must equal the oracle's run for
run; checkpoints of host-resident state saved under one partition and
restored under another must equal the oracle's reshard bit for bit, padding
zero; a restore followed by a step of the native host AdamW must equal the
uninterrupted step; and every way a set of files can be incomplete or damaged
(026 notes §五: a missing process file must fail explicitly) must raise.

Pages cited by short name:
  026 notes  "026｜ZeRO：数据并行中，没必要让每张卡保存全部训练状态" (wq-win.github.io)
"""

import os
import pathlib

import numpy as np
import pytest
import torch

from oracle import partition, rounding
from zero_sharded_mixed_flat_amd import abi

STAGING = abi.ZERO_CKPT_MIN_STAGING


def _plans(units, nd, stage, align):
    return abi.Plan(units, nd, stage, align), partition.make_plan(units, nd, stage, align)


def _staging(nbytes=STAGING):
    return torch.empty(nbytes, dtype=torch.uint8)


def _state(ref_plan, seed):
    """Three fp32 shards per owner cut from random flat vectors (padding zero)."""
    rng = np.random.default_rng(seed)
    flats = [rng.standard_normal(ref_plan.psi).astype(np.float32) for _ in range(3)]
    return flats, [[partition.shard_of(ref_plan, f, r) for f in flats] for r in range(ref_plan.owners)]


def _save_all(tmp_path, plan, shards, step, tag="run"):
    paths = []
    for r, arrays in enumerate(shards):
        path = str(tmp_path / f"{tag}-rank{r:04d}.zck")
        t = [torch.from_numpy(a.copy()) for a in arrays]
        abi.zero_ckpt_save(path, plan, r, step, *t, _staging())
        paths.append(path)
    return paths


def _load(paths, plan, rank, n, staging=None):
    t = [torch.full((n,), float("nan")) for _ in range(3)]
    step = abi.zero_ckpt_load(paths, plan, rank, *t, staging if staging is not None else _staging())
    return step, [x.numpy() for x in t]


@pytest.mark.parametrize("seed", range(25))
def test_runs_match_oracle(seed):
    rng = np.random.default_rng(seed)

    def random_plan(psi=None):
        units = [int(x) for x in rng.integers(0, 5000, int(rng.integers(1, 6)))]
        if psi is not None:
            units[-1] += psi - sum(units)
            if units[-1] < 0:
                units = [psi]
        if sum(units) == 0:
            units[0] = 1
        args = (units, int(rng.integers(1, 40)), int(rng.integers(0, 4)), int(rng.choice([1, 8, 256])))
        return abi.Plan(*args), partition.make_plan(*args)

    old, old_ref = random_plan()
    new, new_ref = random_plan(old_ref.psi)
    for r in range(new_ref.nd):
        assert abi.zero_plan_reshard(old, new, r) == partition.reshard_segments(old_ref, new_ref, r)


def test_runs_rejects():
    a, _ = _plans([1000], 4, 2, 8)
    b, _ = _plans([1001], 4, 2, 8)
    with pytest.raises(abi.ZeroError):
        abi.zero_plan_reshard(a, b, 0)
    with pytest.raises(abi.ZeroError):
        abi.zero_plan_reshard(a, a, 4)


@pytest.mark.parametrize("old_args, new_args", [
    (([70_000, 1234, 99_999], 4, 3, 8), ([70_000, 1234, 99_999], 4, 3, 8)),      # same partition
    (([70_000, 1234, 99_999], 4, 3, 8), ([70_000, 1234, 99_999], 7, 2, 16)),     # Nd and stage change
    (([600_000], 3, 1, 8), ([100_000, 500_000], 16, 3, 256)),                     # layers appear
    (([300_001], 1, 0, 8), ([300_001], 5, 3, 1)),                                 # from plain data parallelism
])
def test_restore_equals_oracle_reshard(tmp_path, old_args, new_args):
    old, old_ref = _plans(*old_args)
    new, new_ref = _plans(*new_args)
    _, shards = _state(old_ref, 1)
    paths = _save_all(tmp_path, old, shards, step=17)
    assert not any(p.endswith(".tmp") for p in os.listdir(tmp_path))
    for r in range(new_ref.nd):
        step, got = _load(paths, new, r, new_ref.shard_numel)
        assert step == 17
        for k in range(3):
            expect = partition.reshard(old_ref, [s[k] for s in shards], new_ref, r)
            assert np.array_equal(got[k].view(np.uint32), expect.view(np.uint32)), (r, k)


def test_round_trip_8_16_8(tmp_path):
    units = [1 << 19, 33, 1 << 18]             # several checksum blocks per shard
    p8, r8 = _plans(units, 8, 3, 8)
    p16, r16 = _plans(units, 16, 3, 8)
    _, shards = _state(r8, 2)
    paths8 = _save_all(tmp_path, p8, shards, step=5, tag="a")
    shards16 = [_load(paths8, p16, r, r16.shard_numel)[1] for r in range(16)]
    paths16 = _save_all(tmp_path, p16, shards16, step=5, tag="b")
    for r in range(8):
        _, back = _load(paths16, p8, r, r8.shard_numel, _staging(3 * STAGING))
        for k in range(3):
            assert np.array_equal(back[k], shards[r][k])


def test_step_after_restore_equals_uninterrupted(tmp_path):
    # One AdamW step at Nd = 4 (host AdamW, the offload path), save, restore at
    # Nd = 6 and step again: the same state and parameters as two steps at Nd = 4.
    units = [50_000, 20_011]
    pa, ra = _plans(units, 4, 3, 8)
    pb, rb = _plans(units, 6, 2, 8)
    flats, shards = _state(ra, 3)
    flats[2] = np.abs(flats[2]) * 1e-6
    shards = [[partition.shard_of(ra, f, r) for f in flats] for r in range(4)]
    rng = np.random.default_rng(4)
    grads = [rounding.narrow((rng.standard_normal(ra.psi) * 1e-3).astype(np.float32), "bf16") for _ in range(2)]

    def adam(ref_plan, shard_state, rank, flat_grad, t):
        g = partition.shard_of(ref_plan, flat_grad, rank)
        p, m, v = (torch.from_numpy(a.copy()) for a in shard_state)
        out = torch.zeros(ref_plan.shard_numel, dtype=torch.int16)
        hp = abi.adam_hparams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, t)
        abi.zero_cpu_adam_step(p, m, v, torch.from_numpy(g.view(np.int16)), "bf16", ref_plan.shard_numel, hp,
                               0.75, False, out, "bf16", 2)
        return [p.numpy(), m.numpy(), v.numpy()]

    after1 = [adam(ra, shards[r], r, grads[0], 1) for r in range(4)]
    straight = [adam(ra, after1[r], r, grads[1], 2) for r in range(4)]
    paths = _save_all(tmp_path, pa, after1, step=1)
    resumed = []
    for r in range(6):
        step, st = _load(paths, pb, r, rb.shard_numel)
        resumed.append(adam(rb, st, r, grads[1], step + 1))
    for k in range(3):
        a = partition.merge(ra, [s[k] for s in straight])
        b = partition.merge(rb, [s[k] for s in resumed])
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_missing_foreign_and_damaged_files(tmp_path):
    plan, ref = _plans([700_000], 4, 1, 8)
    _, shards = _state(ref, 5)
    paths = _save_all(tmp_path, plan, shards, step=3)
    n = ref.shard_numel

    def load_error(paths_, rank=0, plan_=plan, n_=n):
        with pytest.raises(abi.ZeroError) as e:
            _load(paths_, plan_, rank, n_)
        return e.value

    # a process's file is missing: explicit failure naming it, whichever rank restores
    gone = list(paths)
    gone[2] = str(tmp_path / "never-written.zck")
    for rank in range(4):
        e = load_error(gone, rank)
        assert e.code == abi.ZERO_EIO and "rank 2" in str(e) and "never-written" in str(e)
    # too few files, or files in the wrong order
    assert load_error(paths[:3]).code == abi.ZERO_EINVAL
    swapped = [paths[1], paths[0]] + paths[2:]
    assert "holds rank 1" in str(load_error(swapped))
    # a file of another step
    other = _save_all(tmp_path, plan, shards, step=4, tag="later")
    assert load_error(paths[:3] + other[3:]).code == abi.ZERO_EINVAL
    # another model size
    plan2, ref2 = _plans([700_001], 4, 1, 8)
    assert "parameters" in str(load_error(paths, 0, plan2, ref2.shard_numel))
    # truncated
    damaged = str(tmp_path / "damaged.zck")
    data = pathlib.Path(paths[1]).read_bytes()
    pathlib.Path(damaged).write_bytes(data[:-4])
    assert "truncated" in str(load_error([paths[0], damaged] + paths[2:]))
    # one flipped bit in rank 1's m array: rank 1's restore reads it and fails
    header = os.path.getsize(paths[1]) - 3 * 4 * n
    flipped = bytearray(data)
    flipped[header + 4 * n + 4 * 100_000] ^= 0x10                 # m[100000] of a 175000-element shard
    pathlib.Path(damaged).write_bytes(bytes(flipped))
    e = load_error([paths[0], damaged] + paths[2:], rank=1)
    assert e.code == abi.ZERO_EIO and "corrupt" in str(e) and "array 1" in str(e)
    # a damaged header
    flipped = bytearray(data)
    flipped[40] ^= 1
    pathlib.Path(damaged).write_bytes(bytes(flipped))
    assert "corrupt header" in str(load_error([paths[0], damaged] + paths[2:]))
    # not a checkpoint at all
    pathlib.Path(damaged).write_bytes(b"x" * 4096)
    assert "not a checkpoint" in str(load_error([paths[0], damaged] + paths[2:]))


def test_concurrent_saves_to_one_path(tmp_path):
    # Each save writes its own temporary file: eight threads saving different
    # states to one path leave exactly one whole file, equal to one of them.
    import threading
    plan, ref = _plans([50_000], 2, 2, 8)
    n = ref.shard_numel
    path = str(tmp_path / "r0.zck")
    states = [[torch.full((n,), float(k + a)) for a in range(3)] for k in range(8)]
    errors = []

    def save(k):
        try:
            abi.zero_ckpt_save(path, plan, 0, 5, *states[k], _staging())
        except Exception as exc:                                   # noqa: BLE001
            errors.append(exc)

    threads = [threading.Thread(target=save, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors
    assert os.listdir(tmp_path) == ["r0.zck"]                      # no temporary file left behind
    abi.zero_ckpt_save(str(tmp_path / "r1.zck"), plan, 1, 5, *states[0], _staging())
    out = [torch.empty(n) for _ in range(3)]
    assert abi.zero_ckpt_load([path, str(tmp_path / "r1.zck")], plan, 0, *out, _staging()) == 5
    # rank 0's file is exactly one of the eight saves, whole (a torn mix of
    # two would also fail the block checksums)
    assert sum(all(torch.equal(o, st) for o, st in zip(out, states[k])) for k in range(8)) == 1


def test_save_rejects_and_leaves_nothing(tmp_path):
    plan, ref = _plans([1000], 2, 2, 8)
    t = [torch.zeros(ref.shard_numel) for _ in range(3)]
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_ckpt_save(str(tmp_path / "no-such-dir" / "x.zck"), plan, 0, 1, *t, _staging())
    assert e.value.code == abi.ZERO_EIO
    with pytest.raises(abi.ZeroError):
        abi.zero_ckpt_save(str(tmp_path / "x.zck"), plan, 2, 1, *t, _staging())          # rank out of range
    with pytest.raises(abi.ZeroError):
        abi.zero_ckpt_save(str(tmp_path / "x.zck"), plan, 0, 1, *t, _staging(), staging_bytes=STAGING - 64)
    with pytest.raises(ValueError):
        abi.zero_ckpt_save(str(tmp_path / "x.zck"), plan, 0, 1, *t, _staging(1024))
    assert os.listdir(tmp_path) == []
