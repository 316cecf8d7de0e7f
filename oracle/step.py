"""The step itself: reduce, exact norm, clip, Adam(W), cast, gather.

Test infrastructure: see the package docstring.

One rank's share of the step, in the pages' order (CMU 11-868 Lecture 18
notes §2.2, ZeRO-1 walk-through, steps 3-5; ZeRO paper notes 0x05 §5.2):

1. reduce-scatter: the owner receives the AVERAGE gradient of its slice,
   summed over ranks in a fixed rank order (§2.5 of the same notes).
2. gradient clipping by the global L2 norm (L3.2 Memory optimisation and ZeRO
   §4.2 ``gradient_clipping``; Lecture 18 notes §1.4 on norms over the flat
   gradient buffer).
3. the owner updates its fp32 variance, momentum and master, then copies the
   master to the 16-bit parameter.
4. all-gather of the updated 16-bit slices.

Everything is numpy on the CPU.  The reduce is done in float32 (the precision
the method accumulates in); the norm is exact; Adam is evaluated in float64
from the float32 inputs and rounded to float32 once per output.

Pages cited by short name:
  L3.2              "L3.2 显存优化与 ZeRO" (yulong.wang)
  ZeRO paper notes  "ZeRO:" paper notes (puzhiyuan.github.io)
"""

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .partition import shard_of
from .rounding import is_finite16, narrow, widen

_CHUNK = 1 << 24   # elements per exact-sum chunk; keeps every bucket sum below 2**53


@dataclass(frozen=True)
class AdamHparams:
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    inv_loss_scale: float = 1.0
    max_norm: float = 1.0          # <= 0 disables clipping


def _f32(x):
    """The float32 value a device receives for host scalar ``x``, as a Python float."""
    return float(np.float32(x))


# ---------------------------------------------------------------------------
# 1. reduce-scatter, local half
# ---------------------------------------------------------------------------

def reduce_shard(contribs, dtype):
    """Average of the Nd ranks' contributions to one owned slice.

    ``contribs`` is a sequence of Nd uint16 arrays of equal length, rank 0
    first.  The sum runs over ranks 0, 1, ..., Nd-1 in float32 (each addition
    rounded), then one IEEE float32 division by Nd, then round-to-nearest-even
    into the 16-bit dtype.  The loss scale, if any, stays in the stored value.

    Returns (reduced uint16 array, nonfinite) where ``nonfinite`` is True if any
    contribution or any output is inf or NaN.
    """
    contribs = [np.asarray(c, dtype=np.uint16) for c in contribs]
    if not contribs:
        raise ValueError("need at least one contribution")
    n = contribs[0].shape[0]
    if any(c.shape != (n,) for c in contribs):
        raise ValueError("contributions must be 1-D and of equal length")
    acc = widen(contribs[0], dtype).copy()
    for c in contribs[1:]:
        with np.errstate(over="ignore"):       # an overflow to infinity is reported by the flag
            acc = acc + widen(c, dtype)        # float32 + float32 -> float32
    mean = acc / np.float32(len(contribs))     # float32 IEEE division
    out = narrow(mean, dtype)
    nonfinite = not all(bool(np.all(is_finite16(c, dtype))) for c in contribs)
    nonfinite = nonfinite or not bool(np.all(is_finite16(out, dtype)))
    return out, nonfinite


# ---------------------------------------------------------------------------
# 2. global L2 norm and clip coefficient
# ---------------------------------------------------------------------------

def sumsq_exact(bits, dtype, inv_loss_scale=1.0):
    """Exact sum of (value * inv_loss_scale)**2 over a 16-bit array, as a Fraction.

    Each 16-bit value is M * 2**e with an integer |M| < 2**11, so its square is
    M**2 * 2**(2e): summing the integers M**2 per exponent and then adding the
    exponent buckets as Python ints loses nothing.  The result therefore does
    not depend on how the vector is split into ranks or chunks, which is what
    lets a sharded norm equal the unsharded one bit for bit.  Raises
    ValueError on non-finite input (the step is skipped instead).
    """
    scale = float(inv_loss_scale)
    mant, exp = math.frexp(scale)
    if scale <= 0 or mant != 0.5:
        raise ValueError("inv_loss_scale must be a positive power of two")
    bits = np.asarray(bits, dtype=np.uint16)
    if not np.all(is_finite16(bits, dtype)):
        raise ValueError("non-finite gradient")
    total = Fraction(0)
    for lo in range(0, bits.shape[0], _CHUNK):
        x = widen(bits[lo:lo + _CHUNK], dtype).astype(np.float64) * scale  # exact
        m, e = np.frexp(x)                         # x = m * 2**e, 0.5 <= |m| < 1
        big_m = np.ldexp(m, 11)                    # integer valued for 16-bit inputs
        if not np.all(big_m == np.rint(big_m)):
            raise AssertionError("value with more than 11 significant bits")
        sq = big_m * big_m                         # < 2**22, exact
        e2 = 2 * (e.astype(np.int64) - 11)         # x**2 = sq * 2**e2
        if x.size == 0:
            continue
        e_min = int(e2.min())
        buckets = np.bincount(e2 - e_min, weights=sq)   # integer sums < 2**53: exact
        acc = 0
        for k in range(buckets.shape[0] - 1, -1, -1):
            acc = (acc << 1) + int(buckets[k])
        total += Fraction(acc) * (Fraction(2) ** e_min)
    return total


def norm_from_sumsq(sumsq):
    """L2 norm in float64 from an exact sum of squares (one rounding, then sqrt)."""
    return math.sqrt(float(sumsq))


def clip_coef(norm, max_norm):
    """Gradient-clipping multiplier, float32: min(1, max_norm / (norm + 1e-6)).

    ``max_norm <= 0`` disables clipping (multiplier 1).  The 1e-6 guard is the
    common library convention; the pages only give ``gradient_clipping: 1.0``.
    """
    if max_norm <= 0:
        return np.float32(1.0)
    return np.float32(min(1.0, float(max_norm) / (float(norm) + 1e-6)))


# ---------------------------------------------------------------------------
# 3. Adam(W) on the owned fp32 state, then the cast to 16 bits
# ---------------------------------------------------------------------------

def bias_corrections(hp, step):
    """float32 values of 1 - beta1**t and 1 - beta2**t, formed in float64."""
    b1, b2 = _f32(hp.beta1), _f32(hp.beta2)
    return _f32(1.0 - b1 ** step), _f32(1.0 - b2 ** step)


def adam_update(master, m, v, grad_bits, grad_dtype, hp, step, coef, param_dtype):
    """One Adam(W) step on float32 master/m/v; returns new (master, m, v, param_bits).

    Kingma & Ba's update with bias correction and epsilon outside the square
    root, plus decoupled weight decay (Loshchilov & Hutter):

        g  = grad * inv_loss_scale * coef
        m' = b1 m + (1 - b1) g
        v' = b2 v + (1 - b2) g^2
        p' = p - lr * ( (m'/bc1) / (sqrt(v'/bc2) + eps) + wd * p )

    All scalars are the float32 values a device would receive.  The arithmetic
    is float64; m', v' and p' are each rounded to float32 once, and the 16-bit
    parameter is the round-to-nearest-even of float32(p').
    """
    if step < 1:
        raise ValueError("Adam step count starts at 1")
    b1, b2 = _f32(hp.beta1), _f32(hp.beta2)
    omb1, omb2 = _f32(1.0 - b1), _f32(1.0 - b2)
    bc1, bc2 = bias_corrections(hp, step)
    lr, eps, wd = _f32(hp.lr), _f32(hp.eps), _f32(hp.weight_decay)
    inv_s = _f32(hp.inv_loss_scale)
    g = widen(grad_bits, grad_dtype).astype(np.float64) * inv_s * float(np.float32(coef))
    m64 = b1 * np.asarray(m, np.float32).astype(np.float64) + omb1 * g
    v64 = b2 * np.asarray(v, np.float32).astype(np.float64) + omb2 * (g * g)
    p = np.asarray(master, np.float32).astype(np.float64)
    p64 = p - lr * ((m64 / bc1) / (np.sqrt(v64 / bc2) + eps) + wd * p)
    p32 = p64.astype(np.float32)
    return p32, m64.astype(np.float32), v64.astype(np.float32), narrow(p32, param_dtype)


# ---------------------------------------------------------------------------
# 4. gather
# ---------------------------------------------------------------------------

def gather(plan, shards, full, unit_begin=0, unit_end=None):
    """Write every owner's slice of units [unit_begin, unit_end) into ``full``.

    ``shards[r]`` is owner r's shard (``plan.shard_numel`` elements) and
    ``full`` the padded full buffer (``plan.full_numel`` elements); both any
    dtype.  A pure copy: full[base_u + r*s_u + j] = shards[r][shard_base_u + j].
    Returns ``full`` (modified in place).
    """
    if unit_end is None:
        unit_end = len(plan.units)
    if len(shards) != plan.owners:
        raise ValueError("need one shard per owner")
    for u in plan.units[unit_begin:unit_end]:
        for r in range(plan.owners):
            dst = u.full_base + r * u.slice_numel
            full[dst:dst + u.slice_numel] = shards[r][u.shard_base:u.shard_base + u.slice_numel]
    return full


# ---------------------------------------------------------------------------
# The whole step, sharded (every owner emulated) and unsharded
# ---------------------------------------------------------------------------

def step_sharded(plan, local_grads, states, hp, step, grad_dtype, param_dtype):
    """Every owner's share of one step, followed by the gather.

    ``local_grads[r]`` is rank r's full local 16-bit gradient (``plan.psi``
    elements).  ``states[o]`` is owner o's (master, m, v) shard.  Returns a dict
    with the per-owner reduced gradients, the global norm and clip multiplier,
    whether the step was skipped, the new per-owner states and the padded full
    16-bit parameter buffer (padding positions hold the cast of the padded
    master, which stays zero).
    """
    if len(local_grads) != plan.nd:
        raise ValueError("need one local gradient per rank")
    reduced, nonfinite = [], False
    for owner in range(plan.owners):
        contribs = [shard_of(plan, g, owner) for g in local_grads]
        out, bad = reduce_shard(contribs, grad_dtype)
        reduced.append(out)
        nonfinite = nonfinite or bad
    result = {"reduced": reduced, "skipped": nonfinite}
    if nonfinite:
        result.update(norm=float("nan"), coef=np.float32(1.0), states=list(states), full=None)
        return result
    total = Fraction(0)
    for out in reduced:                          # combine exact per-owner partials
        total += sumsq_exact(out, grad_dtype, hp.inv_loss_scale)
    norm = norm_from_sumsq(total)
    coef = clip_coef(norm, hp.max_norm)
    new_states, params = [], []
    for owner in range(plan.owners):
        master, m, v = states[owner]
        p, m2, v2, bits = adam_update(master, m, v, reduced[owner], grad_dtype, hp, step, coef,
                                      param_dtype)
        new_states.append((p, m2, v2))
        params.append(bits)
    full = gather(plan, params, np.zeros(plan.full_numel, dtype=np.uint16))
    result.update(norm=norm, coef=coef, states=new_states, full=full)
    return result


def step_sequence(plan, grads_per_step, states, hp, grad_dtype, param_dtype, first_step=1):
    """Consecutive sharded steps; the step count advances only for applied steps.

    ``grads_per_step[k]`` is the list of every rank's full local gradient for
    step k.  A step with a non-finite gradient is skipped whole: the state
    and the step count stay as they were, so the next update takes the bias
    corrections the skipped one would have taken (the pages give no overflow
    policy; a skipped step is treated as if it had not happened).  Returns
    one step_sharded result per step, each with the step count ``t`` it used.
    """
    t = first_step
    out = []
    for grads in grads_per_step:
        res = step_sharded(plan, grads, states, hp, t, grad_dtype, param_dtype)
        res["t"] = t
        out.append(res)
        if not res["skipped"]:
            states = res["states"]
            t += 1
    return out


def step_unsharded(local_grads, master, m, v, hp, step, grad_dtype, param_dtype):
    """Plain data parallelism: every rank reduces and updates the whole vector.

    Written without any partition: the average over ranks of the full local
    gradients, the norm over the whole averaged gradient, Adam over every
    parameter.  Returns (reduced, norm, coef, skipped, master, m, v, param_bits).
    """
    reduced, nonfinite = reduce_shard(local_grads, grad_dtype)
    if nonfinite:
        return reduced, float("nan"), np.float32(1.0), True, master, m, v, None
    norm = norm_from_sumsq(sumsq_exact(reduced, grad_dtype, hp.inv_loss_scale))
    coef = clip_coef(norm, hp.max_norm)
    p, m2, v2, bits = adam_update(master, m, v, reduced, grad_dtype, hp, step, coef, param_dtype)
    return reduced, norm, coef, False, p, m2, v2, bits
