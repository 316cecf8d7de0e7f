"""The parity bar accepts what it should and nothing more: master, m and v
within 1e-9 + 1e-6 relative (a planted 1.25e-6 relative error, or 1.1e-9 on a
tiny value, fails), a 16-bit parameter one ulp off passes and two fail, and
the bit-identity check catches a single fp32 ulp and an fp32 evaluation of
the update.  The norm's derived bound holds against exact rational sums,
even for chains built so that every addition loses nearly a whole rounding,
and a norm accumulated in fp32 fails it."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import rounding, step
from oracle.step import AdamHparams
from tolerance import (U64, adam_ok, adam_parity, adam_same, coef_ok, norm_chain, norm_ok, norm_rel,
                       param16_ok, within)

HP = AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _b(vals, dt):
    return rounding.narrow(np.asarray(vals, np.float32), dt)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_param_one_ulp_passes_two_fail_at_ordinary_magnitude(dt):
    x = _b([0.02, -0.013, 1.5], dt)
    param16_ok(x, x, dt, "equal")
    param16_ok(x + np.uint16(1), x, dt, "one ulp")
    with pytest.raises(AssertionError):
        param16_ok(x + np.uint16(2), x, dt, "two ulps")


def test_param_across_zero():
    # fp16 across zero: -0 against the smallest subnormal is one ulp in value
    param16_ok(np.uint16([0x8000]), np.uint16([0x0001]), "f16", "-0 vs the smallest subnormal")
    with pytest.raises(AssertionError):
        param16_ok(np.uint16([0x8001]), np.uint16([0x0001]), "f16", "opposite subnormals")


def test_within_relative_and_absolute_parts():
    ref = np.float32([0.02, 1e-12, 0.0, np.inf, np.nan])
    within(ref, ref, "identical")
    within(ref + np.float32([0.02 * 7.5e-7, 9e-10, 9e-10, 0, 0]), ref, "inside")
    for k, d in ((0, 0.02 * 1.25e-6), (1, 1.1e-9), (2, 1.1e-9)):
        bad = ref.copy()
        bad[k] += np.float32(d)
        with pytest.raises(AssertionError):
            within(bad, ref, f"planted at {k}")
    with pytest.raises(AssertionError):
        within(np.float32([0.02, 1e-12, 0.0, 3e38, np.nan]), ref, "inf against a finite value")


def _update_inputs(n=1000, seed=0):
    rng = np.random.default_rng(seed)
    g = _b(rng.standard_normal(n) * 1e-4, "bf16")
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    return g, p, m, v


def test_planted_error_fails():
    g, p, m, v = _update_inputs()
    coef = np.float32(0.7)
    ref = step.adam_update(p, m, v, g, "bf16", HP, 2, coef, "bf16")
    adam_parity(ref, ref, "bf16", "identical")
    k = int(np.argmax(np.abs(p)))
    for which in range(3):
        bad = [a.copy() for a in ref]
        x = float(bad[which][k])
        bad[which][k] = np.float32(x + 1.05 * (1e-9 + 1e-6 * abs(x)))
        with pytest.raises(AssertionError):
            adam_ok(tuple(bad), ref, "bf16", f"planted in output {which}")
    # one fp32 ulp passes the bar but not the bit-identity check
    bad = [a.copy() for a in ref]
    bad[0][k] = np.nextafter(bad[0][k], np.float32(1))
    adam_ok(tuple(bad), ref, "bf16", "one fp32 ulp")
    with pytest.raises(AssertionError):
        adam_same(tuple(bad), ref, "one fp32 ulp")
    adam_parity(tuple(bad), ref, "bf16", "one fp32 ulp, different clip multipliers", same=False)


def test_bit_identity_catches_an_fp32_evaluation():
    # The same update evaluated one fp32 operation at a time (not what the
    # library does) meets the bar on these inputs but not bit identity.
    g, p, m, v = _update_inputs(20_000, 3)
    coef = np.float32(0.7)
    t = 2
    ref = step.adam_update(p, m, v, g, "bf16", HP, t, coef, "bf16")
    f = np.float32
    b1, b2 = f(HP.beta1), f(HP.beta2)
    bc1, bc2 = (f(x) for x in step.bias_corrections(HP, t))
    gg = rounding.widen(g, "bf16") * coef
    m2 = b1 * m + f(1 - float(b1)) * gg
    v2 = b2 * v + f(1 - float(b2)) * (gg * gg)
    p2 = p - f(HP.lr) * ((m2 / bc1) / (np.sqrt(v2 / bc2) + f(HP.eps)) + f(HP.weight_decay) * p)
    fp32 = (p2, m2, v2, rounding.narrow(p2, "bf16"))
    adam_ok(fp32, ref, "bf16", "fp32 evaluation")
    with pytest.raises(AssertionError):
        adam_same(fp32, ref, "fp32 evaluation")


def _serial(x):
    acc = float(x[0])
    for t in x[1:]:
        acc += float(t)
    return acc


@pytest.mark.parametrize("k", [1, 7, 33, 87, 300])
def test_summation_bound_for_nonnegative_terms(k):
    # |S' - S| <= g(k) S for k fp64 additions of nonnegative terms.  The
    # adversarial chain adds k terms just under half an ulp of 1 to 1: every
    # addition rounds the term away, so the error is close to the bound and a
    # bound smaller by a constant factor fails.
    g = Fraction(k * U64) / (1 - Fraction(k * U64))
    rng = np.random.default_rng(k)
    for _ in range(20):
        x = rng.random(k + 1) * np.exp2(rng.integers(-60, 60, k + 1).astype(np.float64))
        exact = sum(Fraction(float(t)) for t in x)
        assert abs(Fraction(_serial(x)) - exact) <= g * exact
    x = np.array([1.0] + [U64 * (1 - 2.0 ** -20)] * k)
    exact = sum(Fraction(float(t)) for t in x)
    err = abs(Fraction(_serial(x)) - exact)
    assert err <= g * exact
    assert err > g * exact / 2


def test_norm_chain_lengths():
    assert norm_chain(1) == 33 + 10 + 27                   # one stage
    assert norm_chain(1, n_extra=2) == 72
    assert norm_chain(20_000_003) == 33 + 10 + (2 + 1 + 13) + 27
    big = 10_937_500_000                                    # the 175e9 / 16-rank owner update
    assert norm_chain(big) == 33 + 10 + (3 + 1 + 13) + 27
    assert 40 * U64 < norm_rel(big) < 1e-14


def test_norm_ok_separates_fp64_from_fp32_accumulation():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1_000_000) * 1e-3).astype(np.float32).astype(np.float64)
    sq = x * x
    exact = sum(Fraction(float(t)) for t in sq)
    ref = float(np.sqrt(float(exact)))
    # numpy's pairwise fp64 sum is a tree about 30 additions deep, shallower
    # than the kernels' (a serial sum over 1e6 terms is not, and may fail).
    norm_ok(np.sqrt(np.sum(sq)), ref, x.size, what="fp64 pairwise")
    acc = np.float32(0)
    for t in sq.astype(np.float32)[:200_000]:
        acc = np.float32(acc + t)
    exact32 = sum(Fraction(float(t)) for t in sq[:200_000])
    with pytest.raises(AssertionError):
        norm_ok(np.sqrt(float(acc)), float(np.sqrt(float(exact32))), 200_000, what="fp32 accumulator")


def test_coef_within_one_fp32_ulp():
    ref = np.float32(0.37)
    up = np.nextafter(ref, np.float32(1))
    coef_ok(up, ref)
    coef_ok(np.nextafter(ref, np.float32(0)), ref)
    with pytest.raises(AssertionError):
        coef_ok(np.nextafter(up, np.float32(1)), ref)
    coef_ok(np.float32(1.0), np.float32(1.0))
