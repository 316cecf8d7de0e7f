"""The derived AdamW tolerances accept the fp32 arithmetic's rounding and
nothing grossly more: a 16-bit parameter two ulps off fails at ordinary
magnitudes; the bounds scale with the operands of each update (so a small
result after cancellation gets an operand-sized bound), and a planted error
of a few hundred fp32 ulps in an ordinary element fails.  The norm bound
holds against exact rational sums, even for chains built so that every
addition loses nearly a whole rounding, and a norm accumulated in fp32 fails
it."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import rounding, step
from oracle.step import AdamHparams
from tolerance import U32, U64, adam_bounds, adam_ok, coef_ok, norm_chain, norm_ok, norm_rel, param16_ok

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


def test_param_within_the_master_bound_near_zero():
    got, ref = _b([3e-10], "bf16"), _b([1e-10], "bf16")
    param16_ok(got, ref, "bf16", "cancellation", master_bound=np.array([2.5e-10]))
    with pytest.raises(AssertionError):
        param16_ok(got, ref, "bf16", "no master bound")
    # fp16 across zero: -0 against the smallest subnormal is one ulp in value
    param16_ok(np.uint16([0x8000]), np.uint16([0x0001]), "f16", "-0 vs the smallest subnormal")
    with pytest.raises(AssertionError):
        param16_ok(np.uint16([0x8001]), np.uint16([0x0001]), "f16", "opposite subnormals")


def test_bounds_scale_with_the_operands():
    # ordinary element: the bound on p is a few dozen ulps of |p|
    g = _b([1e-4, 1e-4], "bf16")
    p = np.float32([0.02, 0.003])
    m = np.float32([1e-5, 1e-4])
    v = np.float32([1e-8, 1e-16])                # the second: tiny v, a large step that nearly cancels p
    bp, bm, bv = adam_bounds(p, m, v, g, "bf16", HP, 1, np.float32(1.0))
    g0 = float(rounding.widen(g, "bf16")[0])
    a = (0.9 * 1e-5 + 0.1 * g0) / 0.1 / (np.sqrt((0.95 * 1e-8 + 0.05 * g0 * g0) / 0.05) + 1e-8)
    assert bp[0] == pytest.approx(24 * U32 * (0.02 + 3e-4 * a + 3e-4 * 0.1 * 0.02), rel=1e-3)
    ref = step.adam_update(p, m, v, g, "bf16", HP, 1, np.float32(1.0), "bf16")
    step_size = abs(float(p[1]) - float(ref[0][1]))
    assert step_size > 1e-3                      # the update is large
    assert bp[1] > 24 * U32 * step_size          # and the bound follows it, not |p'|
    assert bm[0] <= 8 * U32 * 1e-5 and bv[0] <= 16 * U32 * 1e-8


def test_planted_error_fails():
    rng = np.random.default_rng(0)
    n = 1000
    g = _b(rng.standard_normal(n) * 1e-4, "bf16")
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    coef = np.float32(0.7)
    ref = step.adam_update(p, m, v, g, "bf16", HP, 2, coef, "bf16")
    adam_ok(ref, ref, (p, m, v), g, "bf16", HP, 2, coef, "bf16", "identical")
    k = int(np.argmax(np.abs(p)))
    for which in range(3):
        bad = [a.copy() for a in ref]
        bad[which][k] = np.float32(bad[which][k] * (1 + 300 * U32))
        with pytest.raises(AssertionError):
            adam_ok(tuple(bad), ref, (p, m, v), g, "bf16", HP, 2, coef, "bf16", f"planted in output {which}")


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
