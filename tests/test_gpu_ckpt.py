"""Sharded checkpoints of device-resident state (026 notes §五).

Saved from HBM through pinned staging and restored into HBM under the same
or another partition: equal to the oracle's reshard bit for bit with zero
padding; a step after a restore equals the uninterrupted step bit for bit;
state saved from the GPU restores into host memory (ZeRO-Offload) and back.

Pages cited by short name:
  026 notes  "026｜ZeRO：数据并行中，没必要让每张卡保存全部训练状态" (wq-win.github.io)
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import partition
from zero_sharded_mixed_flat_amd import synth, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import abi as _abi
    return _abi


def _note(msg):
    print(msg, flush=True)


def _staging(abi, nbytes=None):
    return torch.empty(nbytes or abi.ZERO_CKPT_MIN_STAGING, dtype=torch.uint8, pin_memory=True)


def _bits32(t):
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("old_args, new_args, staging_mult", [
    (([1 << 20, 4099, 77_777], 4, 3, 8), ([1 << 20, 4099, 77_777], 4, 3, 8), 1),
    (([1 << 20, 4099, 77_777], 4, 3, 8), ([1 << 20, 4099, 77_777], 9, 2, 16), 1),
    (([3_000_001], 2, 1, 8), ([1_000_000, 2_000_001], 8, 3, 256), 6),
])
def test_device_restore_equals_oracle_reshard(abi, tmp_path, old_args, new_args, staging_mult):
    _note(f"ckpt {old_args[1:]} -> {new_args[1:]}")
    old, old_ref = abi.Plan(*old_args), partition.make_plan(*old_args)
    new, new_ref = abi.Plan(*new_args), partition.make_plan(*new_args)
    rng = np.random.default_rng(1)
    flats = [rng.standard_normal(old_ref.psi).astype(np.float32) for _ in range(3)]
    shards = [[partition.shard_of(old_ref, f, r) for f in flats] for r in range(old_ref.owners)]
    staging = _staging(abi, staging_mult * abi.ZERO_CKPT_MIN_STAGING)
    paths = []
    for r, arrays in enumerate(shards):
        dev = [torch.from_numpy(a.copy()).cuda() for a in arrays]
        paths.append(str(tmp_path / f"rank{r}.zck"))
        abi.zero_ckpt_save(paths[-1], old, r, 9, *dev, staging)
    for r in range(new_ref.nd):
        out = [torch.full((new_ref.shard_numel,), float("nan"), device="cuda") for _ in range(3)]
        assert abi.zero_ckpt_load(paths, new, r, *out, staging) == 9
        for k in range(3):
            expect = partition.reshard(old_ref, [s[k] for s in shards], new_ref, r)
            assert np.array_equal(_bits32(out[k]), expect.view(np.uint32)), (r, k)


def test_step_after_restore_equals_uninterrupted(abi, tmp_path):
    # Shrunk LLaMA-3-8B layout, one rank's share: step 1, save, restore into a
    # fresh copy of the workload, then step 2 on both: identical bits.
    from zero_sharded_mixed_flat_amd import runner
    w = dataclasses.replace(workloads.get("llama3_8b_nd8_z2"), psi=8 * 300_001 + 3, units=(8 * 300_001 + 3,))
    a = runner.RankStep(w, seed=4)
    a.step()
    staging = _staging(abi, 4 * abi.ZERO_CKPT_MIN_STAGING)
    # a ZeRO-2 rank's file is its own shard; restoring the same partition reads
    # only this rank's file, but every rank's file must exist, so write them all
    paths = []
    for r in range(w.nd):
        paths.append(str(tmp_path / f"rank{r}.zck"))
        src = (a.master[0], a.m[0], a.v[0]) if r == w.rank else tuple(torch.zeros_like(a.master[0]) for _ in range(3))
        abi.zero_ckpt_save(paths[-1], a.plan, r, a.t - 1, *src, staging)
    b = runner.RankStep(w, seed=4)
    step = abi.zero_ckpt_load(paths, b.plan, w.rank, b.master[0], b.m[0], b.v[0], staging)
    b.t = step + 1
    # The synthetic state of this workload fills the last rank's padding too;
    # a restore sets padding to zero, so compare the real elements.
    _, real = a.plan.rank(w.rank)
    assert real < a.n
    for k, (x, y) in enumerate(zip((a.master, a.m, a.v), (b.master, b.m, b.v))):
        assert np.array_equal(_bits32(x[0, :real]), _bits32(y[0, :real])), k
        assert not y[0, real:].any()
    # step 2's gradients are inputs, not state: give both the same (a's reduce
    # wrote its average in place over its own contribution)
    for x, y in zip(a.contribs(0), b.contribs(0)):
        y.copy_(x)
    a.step()
    b.step()
    torch.cuda.synchronize()
    for k, (x, y) in enumerate(zip((a.master, a.m, a.v), (b.master, b.m, b.v))):
        assert np.array_equal(_bits32(x[0, :real]), _bits32(y[0, :real])), k
    base = w.rank * a.n
    assert np.array_equal(synth.bits(a.full[base:base + real]), synth.bits(b.full[base:base + real]))


def test_all_ranks_reshard_4_to_8_on_device(abi, tmp_path):
    # Every owner of the tiny ZeRO-2 workload after one step, restored as 8
    # ZeRO-3 ranks: the merged state is unchanged bit for bit.
    from zero_sharded_mixed_flat_amd import runner
    w = workloads.get("tiny_nd4_z2")
    run = runner.RankStep(w, seed=2)
    run.step()
    staging = _staging(abi)
    paths = []
    for o in range(w.nd):
        paths.append(str(tmp_path / f"tiny{o}.zck"))
        abi.zero_ckpt_save(paths[-1], run.plan, o, 1, run.master[o], run.m[o], run.v[o], staging)
    old_ref = partition.make_plan(w.units, w.nd, w.stage, w.align)
    new_units = [1 << 18, 3 << 18]
    new, new_ref = abi.Plan(new_units, 8, 3, 8), partition.make_plan(new_units, 8, 3, 8)
    restored = [[], [], []]
    for r in range(8):
        out = [torch.empty(new_ref.shard_numel, device="cuda") for _ in range(3)]
        abi.zero_ckpt_load(paths, new, r, *out, staging)
        for k in range(3):
            restored[k].append(out[k].cpu().numpy())
    for k, t in enumerate((run.master, run.m, run.v)):
        before = partition.merge(old_ref, [t[o].cpu().numpy() for o in range(w.nd)])
        after = partition.merge(new_ref, restored[k])
        assert np.array_equal(before.view(np.uint32), after.view(np.uint32)), k


def test_device_state_restores_into_host_memory_and_back(abi, tmp_path):
    plan_args = ([2_000_003], 3, 2, 8)
    plan, ref = abi.Plan(*plan_args), partition.make_plan(*plan_args)
    rng = np.random.default_rng(8)
    staging = _staging(abi, 2 * abi.ZERO_CKPT_MIN_STAGING)
    flats = [rng.standard_normal(ref.psi).astype(np.float32) for _ in range(3)]
    paths = []
    for r in range(3):
        dev = [torch.from_numpy(partition.shard_of(ref, f, r)).cuda() for f in flats]
        paths.append(str(tmp_path / f"d{r}.zck"))
        abi.zero_ckpt_save(paths[-1], plan, r, 2, *dev, staging)
    host = [torch.empty(ref.shard_numel) for _ in range(3)]
    abi.zero_ckpt_load(paths, plan, 1, *host, staging)
    for k in range(3):
        assert np.array_equal(host[k].numpy(), partition.shard_of(ref, flats[k], 1))
    # and from host memory back to a file and into the device
    abi.zero_ckpt_save(str(tmp_path / "h1.zck"), plan, 1, 2, *host, staging)
    mixed = [paths[0], str(tmp_path / "h1.zck"), paths[2]]
    dev = [torch.empty(ref.shard_numel, device="cuda") for _ in range(3)]
    abi.zero_ckpt_load(mixed, plan, 1, *dev, staging)
    for k in range(3):
        assert np.array_equal(dev[k].cpu().numpy(), host[k].numpy())
