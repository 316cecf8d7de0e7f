"""Pins for oracle.step.

Each test ties the oracle to something other than itself: a hand-worked value,
a closed form, a library routine (math.fsum, torch.optim.AdamW,
torch.nn.utils.clip_grad_norm_), or an invariant the pages state (sharded ==
unsharded, reduce-scatter + all-gather == all-reduce, the rank-local negative
control).
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import partition, rounding, step
from oracle.step import AdamHparams

F16 = "f16"
BF16 = "bf16"


def _f16(vals):
    return rounding.narrow(np.asarray(vals, np.float32), F16)


def _rand16(rng, n, std, dtype):
    return rounding.narrow((rng.standard_normal(n) * std).astype(np.float32), dtype)


# ---------------------------------------------------------------------------
# reduce
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [F16, BF16])
def test_reduce_one_rank_is_identity(dtype):
    rng = np.random.default_rng(0)
    c = _rand16(rng, 4097, 1e-3, dtype)
    out, bad = step.reduce_shard([c], dtype)
    assert not bad and np.array_equal(out, c)


@pytest.mark.parametrize("nd", [2, 3, 4, 5, 8, 64])
def test_reduce_equal_contributions_give_the_value(nd):
    # The mean of nd copies of c is c: the fp32 sum c*k is exact for k <= 64
    # and an 11-bit c, and the division by nd is then exact.
    rng = np.random.default_rng(nd)
    c = _rand16(rng, 1000, 1.0, F16)
    out, _ = step.reduce_shard([c] * nd, F16)
    assert np.array_equal(out, c)


def test_reduce_exact_small_integers():
    # Small integers sum exactly in fp32; their mean over 4 ranks is a multiple
    # of 1/4 below 2048, exactly representable in fp16.  A dropped or doubled
    # rank would change the result.
    rng = np.random.default_rng(7)
    vals = rng.integers(-500, 500, size=(4, 3000))
    contribs = [_f16(v) for v in vals]
    out, _ = step.reduce_shard(contribs, F16)
    expect = [Fraction(int(s), 4) for s in vals.sum(axis=0)]
    got = rounding.widen(out, F16).astype(np.float64)
    assert all(Fraction(g) == e for g, e in zip(got, expect))


def test_reduce_sums_in_rank_order_in_fp32():
    # CMU 11-868 Lecture 18 notes §2.5: the emulation sums in a fixed rank order.
    # Ranks hold 65504, 3*2**-24 and -65504.  In fp32 and in rank order,
    # 65504 + 3*2**-24 rounds back to 65504 (ulp 2**-8), so the sum is 0.  Any
    # other order, or a wider accumulator, keeps the small term: 2**-24.
    big, tiny = 65504.0, 3 * 2.0 ** -24
    c = [_f16([big]), _f16([tiny]), _f16([-big])]
    out, _ = step.reduce_shard(c, F16)
    assert int(out[0]) == 0x0000
    out2, _ = step.reduce_shard([c[0], c[2], c[1]], F16)
    assert int(out2[0]) == 0x0001            # (big - big + tiny) / 3 = 2**-24


def test_reduce_divides_by_nd():
    # Mean, not sum (Lecture 18 notes §2.2 step 3: the AVERAGE gradient).
    c = [_f16([1.0]), _f16([2.0]), _f16([3.0])]
    out, _ = step.reduce_shard(c, F16)
    assert rounding.widen(out, F16)[0] == np.float32(2.0)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_reduce_flags_non_finite(dtype):
    rng = np.random.default_rng(3)
    c = [_rand16(rng, 100, 1e-3, dtype) for _ in range(4)]
    _, bad = step.reduce_shard(c, dtype)
    assert not bad
    inf_bits = 0x7C00 if dtype == F16 else 0x7F80
    c[2] = c[2].copy()
    c[2][17] = inf_bits
    _, bad = step.reduce_shard(c, dtype)
    assert bad


def test_reduce_flags_overflowing_mean():
    # Two finite fp16 maxima average to a finite value; the flag stays clear.
    out, bad = step.reduce_shard([_f16([65504.0]), _f16([65504.0])], F16)
    assert not bad and int(out[0]) == 0x7BFF
    # In bf16 the fp32 sum of two maxima overflows: the output is inf, flagged.
    mx = np.array([0x7F7F], np.uint16)
    out, bad = step.reduce_shard([mx, mx], BF16)
    assert bad


# ---------------------------------------------------------------------------
# norm and clip
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [F16, BF16])
def test_sumsq_matches_fsum(dtype):
    # math.fsum returns the correctly rounded sum of its arguments; every
    # square of a 16-bit value is exact in float64, so the two must agree.
    rng = np.random.default_rng(11)
    for n in (0, 1, 7, 4096, 100_003):
        x = _rand16(rng, n, 1e-3, dtype)
        w = rounding.widen(x, dtype).astype(np.float64)
        assert float(step.sumsq_exact(x, dtype)) == math.fsum((w * w).tolist())


def test_sumsq_with_subnormals_and_loss_scale():
    rng = np.random.default_rng(12)
    x = _rand16(rng, 50_000, 1e-5, F16)        # many fp16 subnormals
    w = rounding.widen(x, F16).astype(np.float64) * 2.0 ** -16
    assert float(step.sumsq_exact(x, F16, 2.0 ** -16)) == math.fsum((w * w).tolist())


def test_norm_closed_form_constant():
    # n copies of c: norm = |c| * sqrt(n); with c = 2**-10 and n = 4**9 the
    # result is exactly 2**-10 * 2**9.
    c = _f16(np.full(4 ** 9, -2.0 ** -10))
    norm = step.norm_from_sumsq(step.sumsq_exact(c, F16))
    assert norm == 2.0 ** -1


def test_sumsq_is_split_invariant():
    rng = np.random.default_rng(13)
    x = _rand16(rng, 30_011, 1e-2, BF16)
    whole = step.sumsq_exact(x, BF16)
    cuts = sorted(rng.choice(np.arange(1, x.size), size=9, replace=False))
    parts = np.split(x, cuts)
    assert sum(step.sumsq_exact(p, BF16) for p in parts) == whole


def test_sumsq_rejects_non_power_of_two_scale_and_nonfinite():
    with pytest.raises(ValueError):
        step.sumsq_exact(_f16([1.0]), F16, 0.3)
    with pytest.raises(ValueError):
        step.sumsq_exact(np.array([0x7C00], np.uint16), F16)


@pytest.mark.parametrize("scale", [0.5, 1.0, 3.0, 50.0])
def test_clip_coef_matches_torch_clip_grad_norm(scale):
    # torch.nn.utils.clip_grad_norm_ multiplies gradients by
    # min(1, max_norm / (total_norm + 1e-6)); compare its factor with ours.
    rng = np.random.default_rng(14)
    g = rng.standard_normal(1000) * scale / math.sqrt(1000)
    p = torch.zeros(1000, dtype=torch.float64, requires_grad=True)
    p.grad = torch.from_numpy(g.copy())
    total = torch.nn.utils.clip_grad_norm_([p], max_norm=1.0)
    factor = float((p.grad / torch.from_numpy(g)).mean())
    ours = step.clip_coef(float(total), 1.0)
    assert float(ours) == pytest.approx(factor, rel=2 ** -23)
    assert float(np.linalg.norm(g)) == pytest.approx(float(total), rel=1e-14)


def test_clip_coef_disabled_and_below_threshold():
    assert step.clip_coef(123.0, 0.0) == np.float32(1.0)
    assert step.clip_coef(0.512, 1.0) == np.float32(1.0)
    assert step.clip_coef(10.0, 1.0) == np.float32(1.0 / (10.0 + 1e-6))


# ---------------------------------------------------------------------------
# Adam
# ---------------------------------------------------------------------------

HP_C1 = AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _close(a, b, rel=1e-6, abs_=1e-9):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= abs_ + rel * np.abs(b))


@pytest.mark.parametrize("hp", [
    HP_C1,
    AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),
    AdamHparams(lr=6e-5, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, inv_loss_scale=2.0 ** -16),
])
def test_adam_matches_torch_adamw(hp):
    # torch.optim.AdamW (decoupled weight decay, bias correction, eps outside
    # the root), run in float64 for 4 steps on the same gradients.
    rng = np.random.default_rng(21)
    n = 2000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    scale = 1.0 / hp.inv_loss_scale
    grads = [_rand16(rng, n, 1e-3 * scale, F16) for _ in range(4)]
    coef = np.float32(0.75)
    tp = torch.tensor(p0.astype(np.float64), requires_grad=True)
    f = lambda x: float(np.float32(x))
    opt = torch.optim.AdamW([tp], lr=f(hp.lr), betas=(f(hp.beta1), f(hp.beta2)), eps=f(hp.eps),
                            weight_decay=f(hp.weight_decay), foreach=False)
    master, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t, g in enumerate(grads, start=1):
        g64 = rounding.widen(g, F16).astype(np.float64) * f(hp.inv_loss_scale) * float(coef)
        tp.grad = torch.from_numpy(g64)
        opt.step()
        master, m, v, bits = step.adam_update(master, m, v, g, F16, hp, t, coef, BF16)
        st = opt.state[tp]
        # The oracle rounds m, v, p to float32 every step while torch keeps
        # float64, so they drift by float32 roundings; where m crosses zero the
        # drift is large only relative to m.  Any error in the formula is of
        # the order of the quantity itself: the absolute slack is 2e-6 of its RMS.
        for ours, ref in ((m, st["exp_avg"]), (v, st["exp_avg_sq"]), (master, tp.detach())):
            ref = ref.numpy()
            rms = float(np.sqrt(np.mean(ref * ref)))
            assert _close(ours, ref, rel=1e-6, abs_=2e-6 * rms)
        assert np.array_equal(bits, rounding.narrow(master, BF16))


def test_adam_first_step_closed_form():
    # From m = v = 0 at t = 1: m_hat = g and v_hat = g**2, so
    # p1 = p0 - lr * (g / (|g| + eps) + wd * p0).
    rng = np.random.default_rng(22)
    n = 5000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = _rand16(rng, n, 1e-3, F16)
    zeros = np.zeros(n, np.float32)
    p1, m1, v1, _ = step.adam_update(p0, zeros, zeros, g, F16, HP_C1, 1, np.float32(1.0), F16)
    gv = rounding.widen(g, F16).astype(np.float64)
    lr, wd, eps = float(np.float32(3e-4)), float(np.float32(0.1)), float(np.float32(1e-8))
    expect = p0.astype(np.float64) - lr * (gv / (np.abs(gv) + eps) + wd * p0.astype(np.float64))
    assert _close(p1, expect, rel=2e-7, abs_=1e-12)
    # m1 = (1 - beta1) * g with beta1 the float32 value of 0.9; 1 - f32(0.9) is
    # exact (Sterbenz) and is 0.100000024, not f32(0.1).
    assert _close(m1, (1.0 - float(np.float32(0.9))) * gv, rel=1e-7, abs_=0)


def test_adam_constant_gradient_many_steps():
    # With a constant gradient g, bias correction makes m_hat = g and
    # v_hat = g**2 at every step, so each step moves p by lr * g / (|g| + eps)
    # exactly (wd = 0).  A wrong bias correction breaks this after step 1.
    hp = AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    g = _f16([1e-3, -2e-2, 5.0, -7e-6])
    gv = rounding.widen(g, F16).astype(np.float64)
    p = np.array([0.5, -0.25, 0.125, 1.0], np.float32)
    m = v = np.zeros(4, np.float32)
    p_ref = p.astype(np.float64)
    lr, eps = float(np.float32(1e-3)), float(np.float32(1e-8))
    for t in range(1, 11):
        p, m, v, _ = step.adam_update(p, m, v, g, F16, hp, t, np.float32(1.0), F16)
        p_ref = p_ref - lr * gv / (np.abs(gv) + eps)
    assert _close(p, p_ref, rel=1e-6, abs_=1e-8)


def test_adam_weight_decay_only():
    # Zero gradient: m = v = 0, the Adam term is 0 / (0 + eps) = 0, and
    # decoupled weight decay gives p_t = p0 * (1 - lr * wd)**t.
    p0 = np.array([0.02, -1.5, 3.0], np.float32)
    zeros = np.zeros(3, np.float32)
    g = np.zeros(3, np.uint16)
    p, m, v = p0, zeros, zeros
    for t in range(1, 6):
        p, m, v, _ = step.adam_update(p, m, v, g, BF16, HP_C1, t, np.float32(1.0), BF16)
    lr, wd = float(np.float32(3e-4)), float(np.float32(0.1))
    assert _close(p, p0.astype(np.float64) * (1 - lr * wd) ** 5, rel=1e-6, abs_=0)
    assert np.all(m == 0) and np.all(v == 0)


def test_adam_clip_coefficient_scales_first_moment():
    rng = np.random.default_rng(23)
    g = _rand16(rng, 64, 1e-2, F16)
    z = np.zeros(64, np.float32)
    _, m_a, _, _ = step.adam_update(z, z, z, g, F16, HP_C1, 1, np.float32(1.0), F16)
    _, m_b, _, _ = step.adam_update(z, z, z, g, F16, HP_C1, 1, np.float32(0.5), F16)
    assert np.array_equal(m_b, (m_a.astype(np.float64) * 0.5).astype(np.float32))


# ---------------------------------------------------------------------------
# the whole step: sharded == unsharded, and the negative control
# ---------------------------------------------------------------------------

def _setup(psi, nd, seed, dtype=F16, std=1e-3):
    rng = np.random.default_rng(seed)
    local = [_rand16(rng, psi, std, dtype) for _ in range(nd)]
    master = (rng.standard_normal(psi) * 0.02).astype(np.float32)
    m = (rng.standard_normal(psi) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(psi) * 1e-8).astype(np.float32)
    return local, master, m, v


@pytest.mark.parametrize("nd", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("stage", [1, 2, 3])
def test_sharded_equals_unsharded(nd, stage):
    # CMU 11-868 Lecture 18 notes §2.5: trained parameters are bit-identical to
    # data parallelism in a fixed-rank-order emulation.
    units = [1001, 37, 2050] if stage == 3 else [3088]
    psi = sum(units)
    local, master, m, v = _setup(psi, nd, seed=100 * nd + stage)
    hp = AdamHparams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=0.01)
    plan = partition.make_plan(units, nd, stage, align=8)
    states = [tuple(partition.shard_of(plan, a, r) for a in (master, m, v)) for r in range(plan.owners)]
    res = step.step_sharded(plan, local, states, hp, 1, F16, F16)
    red, norm, coef, skipped, p, m2, v2, bits = step.step_unsharded(local, master, m, v, hp, 1, F16, F16)
    assert not skipped and not res["skipped"]
    assert res["norm"] == norm and res["coef"] == coef and coef < 1.0   # clipping active
    assert np.array_equal(partition.unpad(plan, res["full"]), bits)
    for r in range(plan.owners):
        for got, ref in zip(res["states"][r], (p, m2, v2)):
            assert np.array_equal(got, partition.shard_of(plan, ref, r))
        assert np.array_equal(res["reduced"][r], partition.shard_of(plan, red, r))


def test_reduce_scatter_then_gather_is_all_reduce():
    # Lecture 18 notes §2.2 and exercise 3: all-reduce = reduce-scatter +
    # all-gather.  Gathering every owner's averaged slice gives the averaged
    # full vector.
    psi, nd = 1 << 12, 4
    local, *_ = _setup(psi, nd, seed=5)
    plan = partition.make_plan([psi], nd, 2)
    slices = []
    for r in range(nd):
        out, _ = step.reduce_shard([partition.shard_of(plan, g, r) for g in local], F16)
        slices.append(out)
    full = step.gather(plan, slices, np.zeros(plan.full_numel, np.uint16))
    allreduce, _ = step.reduce_shard(local, F16)
    assert np.array_equal(partition.unpad(plan, full), allreduce)


def test_rank_local_update_differs():
    # ZeRO reading notes 026 §三: updating a block with only the owner's local
    # gradient changes the algorithm; the result must differ.
    psi, nd = 4096, 4
    local, master, m, v = _setup(psi, nd, seed=6)
    plan = partition.make_plan([psi], nd, 2)
    hp = AdamHparams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, max_norm=0.0)
    states = [tuple(partition.shard_of(plan, a, r) for a in (master, m, v)) for r in range(nd)]
    good = step.step_sharded(plan, local, states, hp, 1, F16, F16)
    for r in range(nd):
        own_only, _ = step.reduce_shard([partition.shard_of(plan, local[r], r)], F16)
        assert not np.array_equal(own_only, good["reduced"][r])
        p_bad, *_ = step.adam_update(*states[r], own_only, F16, hp, 1, np.float32(1.0), F16)
        assert not np.array_equal(p_bad, good["states"][r][0])


def test_non_finite_skips_the_whole_step():
    psi, nd = 2048, 4
    local, master, m, v = _setup(psi, nd, seed=8)
    local[1] = local[1].copy()
    local[1][999] = 0x7E00          # NaN in one rank's gradient
    plan = partition.make_plan([psi], nd, 2)
    states = [tuple(partition.shard_of(plan, a, r) for a in (master, m, v)) for r in range(nd)]
    res = step.step_sharded(plan, local, states, HP_C1, 1, F16, F16)
    assert res["skipped"] and res["full"] is None
    for r in range(nd):
        for got, ref in zip(res["states"][r], states[r]):
            assert got is ref


def test_skipped_step_is_as_if_it_never_happened():
    # Three steps with a NaN in the second: the third update equals the second
    # of a run without the bad step (same state, same step count t = 2), and
    # differs from an update that took t = 3 (the bias corrections matter).
    psi, nd = 2048, 4
    plan = partition.make_plan([psi], nd, 2)
    rng = np.random.default_rng(18)
    grads = [[_rand16(rng, psi, 1e-3, F16) for _ in range(nd)] for _ in range(3)]
    grads[1][2] = grads[1][2].copy()
    grads[1][2][77] = 0x7C00        # +inf in one rank's gradient of step 2
    _, master, m, v = _setup(psi, nd, seed=19)
    states = [tuple(partition.shard_of(plan, a, r) for a in (master, m, v)) for r in range(nd)]
    hp = AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_norm=1.0)
    run = step.step_sequence(plan, grads, states, hp, F16, F16)
    assert [r["t"] for r in run] == [1, 2, 2] and [r["skipped"] for r in run] == [False, True, False]
    clean = step.step_sequence(plan, [grads[0], grads[2]], states, hp, F16, F16)
    assert np.array_equal(run[2]["full"], clean[1]["full"])
    for a, b in zip(run[2]["states"], clean[1]["states"]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    advanced = step.step_sharded(plan, grads[2], run[0]["states"], hp, 3, F16, F16)
    assert not np.array_equal(advanced["full"], run[2]["full"])


def test_padding_stays_zero():
    # Padded positions carry zero gradient and zero state; Adam keeps them 0.
    units, nd = [1000], 16       # slice 64, 1024 padded, 24 padding elements
    local, master, m, v = _setup(sum(units), nd, seed=9)
    plan = partition.make_plan(units, nd, 2)
    states = [tuple(partition.shard_of(plan, a, r) for a in (master, m, v)) for r in range(nd)]
    res = step.step_sharded(plan, local, states, HP_C1, 3, F16, F16)
    p15 = res["states"][15][0]
    assert plan.real_numel(15) == 40 and np.all(p15[40:] == 0)
    assert np.all(res["full"][1000:] == 0)
