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
