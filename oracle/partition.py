"""Flat-bucket partition: which padded positions each data-parallel rank owns.

Test infrastructure: see the package docstring.

Pages:
* Adam is elementwise, so the parameter vector can be cut into Nd pieces and
  rank r keeps only piece r's optimizer state (CMU 11-868 Lecture 18 notes §2.1).
* DeepSpeed concatenates all parameters into one flat vector and cuts it into
  Nd equal pieces, so one tensor may straddle two ranks (Lecture 18 notes §3.2;
  exercise 6 answer: sizes 100/60/40 on 2 ranks give 100 and 100).
* ZeRO-3 flattens and splits per module, and gathers one module's parameters
  into a contiguous buffer (Illustrated distributed training (8) ZeRO §8.4);
  FSDP's unit is usually one transformer layer (Lecture 18 notes §3.3).

Readings (the pages never mention padding or per-stage layout):
* stages 1 and 2 use ONE unit, the whole flat vector; stage 3 partitions each
  unit (layer) separately; stage 0 is plain data parallelism, where every rank
  owns everything.
* the slice of a unit of U elements is s = roundup(ceil(U / Nd), align); rank r
  owns unit-local padded positions [r*s, (r+1)*s).  Positions >= U are padding.
* a unit's base in the padded full buffer is the sum of the padded sizes of
  the units before it; its base inside every rank's shard is the sum of the
  slices before it.

Everything here is exact integer arithmetic on Python ints.

Pages cited by short name:
  026 notes  "026｜ZeRO：数据并行中，没必要让每张卡保存全部训练状态" (wq-win.github.io)
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Unit:
    numel: int        # real elements U in this unit
    slice_numel: int  # s: elements each owner holds for this unit (padded)
    full_base: int    # first position of this unit in the padded full buffer
    shard_base: int   # first position of this unit's slice inside a rank's shard


@dataclass(frozen=True)
class Plan:
    nd: int
    stage: int
    align: int
    units: tuple
    owners: int       # number of distinct owners (1 for stage 0, else nd)

    @property
    def shard_numel(self):
        return sum(u.slice_numel for u in self.units)

    @property
    def full_numel(self):
        return sum(self.owners * u.slice_numel for u in self.units)

    @property
    def psi(self):
        return sum(u.numel for u in self.units)

    def owned(self, rank, unit_index):
        """Unit-local real positions [lo, hi) owned by ``rank`` (hi may equal lo)."""
        u = self.units[unit_index]
        r = 0 if self.owners == 1 else rank
        lo = min(r * u.slice_numel, u.numel)
        hi = min((r + 1) * u.slice_numel, u.numel)
        return lo, hi

    def real_numel(self, rank):
        total = 0
        for i in range(len(self.units)):
            lo, hi = self.owned(rank, i)
            total += hi - lo
        return total


def _ceil_div(a, b):
    return -(-a // b)


def make_plan(unit_numels, nd, stage, align=8):
    """Partition ``unit_numels`` over ``nd`` ranks for a ZeRO ``stage`` in {0,1,2,3}."""
    unit_numels = [int(x) for x in unit_numels]
    if not (1 <= nd <= 1024):
        raise ValueError("nd must be in [1, 1024]")
    if stage not in (0, 1, 2, 3):
        raise ValueError("stage must be 0, 1, 2 or 3")
    if align < 1:
        raise ValueError("align must be >= 1")
    if not unit_numels or any(x < 0 for x in unit_numels):
        raise ValueError("need at least one unit, all sizes >= 0")
    if stage != 3:
        unit_numels = [sum(unit_numels)]
    owners = 1 if stage == 0 else nd
    units, full_base, shard_base = [], 0, 0
    for numel in unit_numels:
        s = _ceil_div(_ceil_div(numel, owners), align) * align
        units.append(Unit(numel, s, full_base, shard_base))
        full_base += owners * s
        shard_base += s
    return Plan(nd, stage, align, tuple(units), owners)


def segments(plan, tensor_numels, rank):
    """Pieces of the named tensors that ``rank`` owns, in shard order.

    Tensors are laid out back to back: for stages 0-2 across the one flat unit,
    for stage 3 filling the units in order (a tensor may not cross a unit).
    Returns a list of (tensor, tensor_offset, shard_offset, length).
    """
    tensor_numels = [int(x) for x in tensor_numels]
    # Assign each tensor its unit and unit-local start.
    placed, unit_i, pos = [], 0, 0
    for t, numel in enumerate(tensor_numels):
        while unit_i < len(plan.units) and pos == plan.units[unit_i].numel and numel > 0:
            unit_i, pos = unit_i + 1, 0
        if unit_i >= len(plan.units) or pos + numel > plan.units[unit_i].numel:
            raise ValueError("tensor sizes do not fill the plan's units")
        placed.append((t, unit_i, pos, numel))
        pos += numel
    if sum(tensor_numels) != plan.psi:
        raise ValueError("tensor sizes do not add up to the plan's parameter count")
    out = []
    for t, ui, start, numel in placed:
        lo, hi = plan.owned(rank, ui)
        a, b = max(lo, start), min(hi, start + numel)
        if a < b:
            u = plan.units[ui]
            r = 0 if plan.owners == 1 else rank
            out.append((t, a - start, u.shard_base + (a - r * u.slice_numel), b - a))
    return out


def shard_of(plan, full_vector, rank):
    """Rank's shard cut out of an UNPADDED flat vector of ``plan.psi`` elements.

    Padding positions are zero.  Works for any numpy dtype.
    """
    full_vector = np.asarray(full_vector)
    if full_vector.shape != (plan.psi,):
        raise ValueError("full_vector must hold exactly psi elements")
    out = np.zeros(plan.shard_numel, dtype=full_vector.dtype)
    flat_base = 0
    for i, u in enumerate(plan.units):
        lo, hi = plan.owned(rank, i)
        r = 0 if plan.owners == 1 else rank
        dst = u.shard_base + (lo - r * u.slice_numel)
        out[dst:dst + (hi - lo)] = full_vector[flat_base + lo:flat_base + hi]
        flat_base += u.numel
    return out


def unpad(plan, padded_full):
    """Real parameters (length psi) out of a padded full buffer (length full_numel)."""
    padded_full = np.asarray(padded_full)
    if padded_full.shape != (plan.full_numel,):
        raise ValueError("padded_full must hold exactly full_numel elements")
    return np.concatenate([padded_full[u.full_base:u.full_base + u.numel] for u in plan.units]) \
        if plan.units else padded_full[:0]


# ---------------------------------------------------------------------------
# Resharding (restoring sharded state under a different partition)
# ---------------------------------------------------------------------------
#
# Pages: a checkpoint of sharded training holds each process's local slice of
# the weights and optimizer state; restoring under a different degree of
# parallelism has to re-own the state while keeping the parameter order and
# which moment belongs to which parameter (026 notes §五).  Reading taken:
# the flat parameter order (units concatenated) is the identity of a
# parameter, so a restore is "merge every old shard into the flat vector, then
# cut the new rank's shard out of it"; padding positions are zero.

def merge(plan, shards):
    """The unpadded flat vector (length psi) held by a complete set of shards."""
    if len(shards) != plan.owners:
        raise ValueError(f"need {plan.owners} shards, got {len(shards)}")
    out = np.zeros(plan.psi, dtype=np.asarray(shards[0]).dtype)
    flat_base = 0
    for i, u in enumerate(plan.units):
        for r in range(plan.owners):
            lo, hi = plan.owned(r, i)
            src = u.shard_base + (lo - r * u.slice_numel)
            out[flat_base + lo:flat_base + hi] = np.asarray(shards[r])[src:src + (hi - lo)]
        flat_base += u.numel
    return out


def reshard(old_plan, old_shards, new_plan, rank):
    """Rank's shard under ``new_plan`` of the state held by ``old_shards`` under ``old_plan``."""
    if old_plan.psi != new_plan.psi:
        raise ValueError("the plans partition different parameter counts")
    return shard_of(new_plan, merge(old_plan, old_shards), rank)


def reshard_segments(old_plan, new_plan, rank):
    """Where each element of rank's new shard comes from, as maximal runs.

    Element by element: position j of the new shard holds flat parameter g (or
    is padding); g lives in old owner r at old shard offset k.  Consecutive j
    with the same r and consecutive k form one run (old_rank, old_offset,
    new_offset, length), in new-shard order.  Padding is in no run.
    """
    if old_plan.psi != new_plan.psi:
        raise ValueError("the plans partition different parameter counts")
    # flat index -> (old owner, old shard offset), one element at a time
    src_rank = np.empty(old_plan.psi, np.int64)
    src_off = np.empty(old_plan.psi, np.int64)
    flat_base = 0
    for i, u in enumerate(old_plan.units):
        for g in range(u.numel):
            r = 0 if old_plan.owners == 1 else g // u.slice_numel
            src_rank[flat_base + g] = r
            src_off[flat_base + g] = u.shard_base + g - r * u.slice_numel
        flat_base += u.numel
    runs = []
    flat_base = 0
    for i, u in enumerate(new_plan.units):
        lo, hi = new_plan.owned(rank, i)
        r_new = 0 if new_plan.owners == 1 else rank
        for g in range(lo, hi):
            j = u.shard_base + g - r_new * u.slice_numel
            r, k = int(src_rank[flat_base + g]), int(src_off[flat_base + g])
            if runs and runs[-1][0] == r and runs[-1][1] + runs[-1][3] == k and runs[-1][2] + runs[-1][3] == j:
                runs[-1][3] += 1
            else:
                runs.append([r, k, j, 1])
        flat_base += u.numel
    return [tuple(x) for x in runs]
