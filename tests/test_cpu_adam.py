"""The native host AdamW of ZeRO-Offload (``zero_cpu_adam_step``) against the oracle.

Runs on the CPU: the update is host code in the same library as the kernels.
The state and the 16-bit parameters are compared with the oracle's fp64
AdamW at the parity bar and bit for bit (the host AdamW evaluates the update
in fp64 in the oracle's order and rounds once, as the GPU kernel does); the
16-bit conversions are pinned exactly (every fp16 pattern widened, fp32
values across the whole fp16/bf16 range narrowed against numpy's
round-to-nearest-even), and every instruction set the CPU offers gives the
oracle's bits, edge values included.
"""

import numpy as np
import pytest
import torch

from oracle import rounding, step
from oracle.step import AdamHparams
from zero_sharded_mixed_flat_amd import abi

from adam_inputs import edge_inputs
from tolerance import adam_parity

HPARAMS = {
    "adam": AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),
    "adamw": AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1),
    "scaled": AdamHparams(lr=6e-5, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.01, inv_loss_scale=2.0 ** -16),
}
ISAS = [i for i in (abi.ZERO_CPU_SCALAR, abi.ZERO_CPU_AVX2, abi.ZERO_CPU_AVX512) if i <= abi.zero_cpu_isa()]


@pytest.fixture(autouse=True)
def _restore_isa():
    isa = abi.zero_cpu_isa()
    yield
    abi.zero_cpu_set_isa(isa)


def _abi_hp(hp, t):
    return abi.adam_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.inv_loss_scale, t)


def _inputs(n, gdt, hp, seed):
    rng = np.random.default_rng(seed)
    scale = 1.0 / hp.inv_loss_scale
    g = rounding.narrow((rng.standard_normal(n) * 1e-3 * scale).astype(np.float32), gdt)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    return g, p, m, v


def _run(g, p, m, v, gdt, pdt, hp, t, coef, threads, skip=False):
    n = g.size
    tp, tm, tv = (torch.from_numpy(a.copy()) for a in (p, m, v))
    tg = torch.from_numpy(g.view(np.int16).copy())
    out = torch.zeros(n, dtype=torch.int16)
    abi.zero_cpu_adam_step(tp, tm, tv, tg, gdt, n, _abi_hp(hp, t), coef, skip, out, pdt, threads)
    return tp.numpy(), tm.numpy(), tv.numpy(), out.numpy().view(np.uint16)


@pytest.mark.parametrize("gdt, pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("hp_name", sorted(HPARAMS))
@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 100_003])
def test_matches_oracle(gdt, pdt, hp_name, n):
    hp = HPARAMS[hp_name]
    g, p, m, v = _inputs(n, gdt, hp, n)
    for t, coef in ((1, 1.0), (7, 0.37)):
        got = _run(g, p, m, v, gdt, pdt, hp, t, coef, threads=3)
        ref = step.adam_update(p, m, v, g, gdt, hp, t, np.float32(coef), pdt)
        adam_parity(got, ref, pdt, f"t={t}")


@pytest.mark.parametrize("gdt, pdt", [("f16", "f16"), ("bf16", "bf16")])
def test_five_steps_each_side_on_its_own_state(gdt, pdt):
    # The host AdamW and the oracle each step from their own previous state;
    # every step must meet the bar, and the two sequences stay bit-identical.
    hp = HPARAMS["adamw"]
    n = 200_003
    rng = np.random.default_rng(12)
    _, p, m, v = _inputs(n, gdt, hp, 12)
    host = (p, m, v)
    for t in range(1, 6):
        g = rounding.narrow((rng.standard_normal(n) * 1e-3).astype(np.float32), gdt)
        coef = np.float32(0.9)
        got = _run(g, *host, gdt, pdt, hp, t, coef, threads=4)
        ref = step.adam_update(p, m, v, g, gdt, hp, t, coef, pdt)
        adam_parity(got, ref, pdt, f"t={t}")
        host = got[:3]
        p, m, v = ref[:3]


@pytest.mark.parametrize("gdt, pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("hp_name", sorted(HPARAMS))
def test_every_isa_gives_the_oracle_bits_on_edge_inputs(gdt, pdt, hp_name):
    # Zeros, fp32 and 16-bit subnormals, gradients whose square overflows fp32:
    # no fused multiply-add, correctly rounded division and square root, one
    # rounding per output, on every instruction set.
    hp = HPARAMS[hp_name]
    g, p, m, v = edge_inputs(50_003, gdt, hp.inv_loss_scale, 21)
    for t, coef in ((1, 1.0), (5, 0.37)):
        with np.errstate(over="ignore"):
            ref = step.adam_update(p, m, v, g, gdt, hp, t, np.float32(coef), pdt)
        for isa in ISAS:
            abi.zero_cpu_set_isa(isa)
            got = _run(g, p, m, v, gdt, pdt, hp, t, coef, threads=3)
            adam_parity(got, ref, pdt, f"isa {isa} t={t}")


def test_consts_fill_gives_the_oracle_scalars():
    # The device kernel's scalars (zero_adam_consts_fill is host code) are the
    # fp32 values the oracle's update takes.
    f32 = lambda x: np.float32(x)
    for hp in HPARAMS.values():
        for t in (1, 2, 10, 1000, 10 ** 6):
            got = abi.zero_adam_consts_fill(_abi_hp(hp, t))
            b1, b2 = float(f32(hp.beta1)), float(f32(hp.beta2))
            bc1, bc2 = step.bias_corrections(hp, t)
            ref = {"lr": f32(hp.lr), "beta1": f32(b1), "beta2": f32(b2), "one_minus_beta1": f32(1.0 - b1),
                   "one_minus_beta2": f32(1.0 - b2), "eps": f32(hp.eps), "weight_decay": f32(hp.weight_decay),
                   "inv_loss_scale": f32(hp.inv_loss_scale), "bias_corr1": f32(bc1), "bias_corr2": f32(bc2)}
            assert sorted(ref) == sorted(name for name, _ in abi.zero_adam_consts._fields_)
            for name, _ in abi.zero_adam_consts._fields_:
                assert np.float32(getattr(got, name)).view(np.uint32) == ref[name].view(np.uint32), (name, t)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_widening_every_pattern_exact(dt):
    # beta1 = 0: m becomes exactly 0*m + f32(grad), for every finite 16-bit pattern.
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    pats = pats[rounding.is_finite16(pats, dt)]
    n = pats.size
    hp = AdamHparams(lr=0.0, beta1=0.0, beta2=0.5, eps=1.0, weight_decay=0.0)
    for isa in ISAS:
        abi.zero_cpu_set_isa(isa)
        _, m, _, _ = _run(pats, np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32),
                          dt, dt, hp, 1, 1.0, threads=2)
        expect = np.float32(0.0) + rounding.widen(pats, dt)       # 0*m + g: -0 becomes +0
        assert np.array_equal(m.view(np.uint32), expect.view(np.uint32)), f"isa {isa}"


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_narrowing_across_the_range_exact(dt):
    # lr = 0 leaves the master unchanged, so the parameter is RNE(master): fp32
    # values over every binade from far below the smallest subnormal to beyond
    # the largest finite value, plus exact ties.
    rng = np.random.default_rng(1)
    exps = rng.integers(-40, 20, 200_000) if dt == "f16" else rng.integers(-140, 128, 200_000)
    x = (rng.uniform(1, 2, exps.size) * np.exp2(exps.astype(np.float64))).astype(np.float32)
    x[::2] *= -1
    if dt == "f16":       # midpoints between neighbouring fp16 values (exact in fp32)
        lo = rounding.widen(np.arange(0, 0x7BFF, 7, dtype=np.uint16), "f16").astype(np.float64)
        hi = rounding.widen(np.arange(1, 0x7C00, 7, dtype=np.uint16), "f16").astype(np.float64)
        ties = ((lo + hi) / 2).astype(np.float32)
    else:                 # bf16 pattern b followed by half an ulp
        ties = ((np.arange(0, 0x7F80, 7, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 65504, 65519.99, 65520, 1e-8])])
    n = x.size
    hp = AdamHparams(lr=0.0, beta1=0.9, beta2=0.9, eps=1.0, weight_decay=0.0)
    zeros16 = np.zeros(n, np.uint16)
    for isa in ISAS:
        abi.zero_cpu_set_isa(isa)
        p, _, _, out = _run(zeros16, x, np.zeros(n, np.float32), np.zeros(n, np.float32), dt, dt, hp, 1, 1.0,
                            threads=2)
        assert np.array_equal(p, x)
        assert np.array_equal(out, rounding.narrow(x, dt)), f"isa {isa}"


@pytest.mark.parametrize("gdt, pdt", [("f16", "f16"), ("bf16", "bf16")])
def test_every_isa_and_thread_count_same_bits(gdt, pdt):
    hp = HPARAMS["adamw"]
    g, p, m, v = _inputs(300_007, gdt, hp, 3)
    p[:1000] *= 1e-6                                 # fp16 subnormal parameters
    abi.zero_cpu_set_isa(abi.ZERO_CPU_SCALAR)
    ref = _run(g, p, m, v, gdt, pdt, hp, 3, 0.5, threads=1)
    for isa in ISAS:
        abi.zero_cpu_set_isa(isa)
        for threads in (1, 4, 16):
            got = _run(g, p, m, v, gdt, pdt, hp, 3, 0.5, threads=threads)
            for a, b in zip(got, ref):
                assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b), (isa, threads)


@pytest.mark.parametrize("offset", [1, 3, 8])
def test_misaligned_output_same_bits(offset):
    # The 16-bit output is streamed when aligned and stored plainly otherwise;
    # an output that starts `offset` elements into a buffer gives the same bits.
    hp = HPARAMS["adamw"]
    n = 100_003
    g, p, m, v = _inputs(n, "bf16", hp, 31)
    ref = _run(g, p, m, v, "bf16", "bf16", hp, 2, 0.7, threads=4)
    for isa in ISAS:
        abi.zero_cpu_set_isa(isa)
        tp, tm, tv = (torch.from_numpy(a.copy()) for a in (p, m, v))
        buf = torch.zeros(n + offset, dtype=torch.int16)
        abi.zero_cpu_adam_step(tp, tm, tv, torch.from_numpy(g.view(np.int16).copy()), "bf16", n, _abi_hp(hp, 2),
                               0.7, False, buf[offset:], "bf16", 4)
        assert np.array_equal(buf[offset:].numpy().view(np.uint16), ref[3]), (isa, offset)
        assert not buf[:offset].any()
        assert np.array_equal(tp.numpy().view(np.uint32), ref[0].view(np.uint32))


def test_skip_writes_nothing():
    hp = HPARAMS["adam"]
    g, p, m, v = _inputs(1000, "f16", hp, 9)
    got = _run(g, p, m, v, "f16", "f16", hp, 1, 1.0, threads=2, skip=True)
    assert np.array_equal(got[0], p) and np.array_equal(got[1], m) and np.array_equal(got[2], v)
    assert not got[3].any()


def test_rejects():
    hp = _abi_hp(HPARAMS["adam"], 1)
    t = [torch.zeros(64) for _ in range(3)]
    g16, out = torch.zeros(64, dtype=torch.int16), torch.zeros(64, dtype=torch.int16)
    cases = [
        (dict(n_threads=0), abi.ZERO_EINVAL),
        (dict(n_threads=257), abi.ZERO_EINVAL),
        (dict(grad_dtype=3), abi.ZERO_EINVAL),
        (dict(coef=0.0), abi.ZERO_EINVAL),
        (dict(coef=float("nan")), abi.ZERO_EINVAL),
        (dict(m=t[0]), abi.ZERO_EALIAS),
        (dict(param_out=g16), abi.ZERO_EALIAS),
        (dict(master=0), abi.ZERO_EINVAL),
    ]
    for over, code in cases:
        args = dict(master=t[0], m=t[1], v=t[2], grad=g16, grad_dtype="f16", n=64, hp=hp, coef=1.0, skip=False,
                    param_out=out, param_dtype="f16", n_threads=2)
        args.update(over)
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_cpu_adam_step(**args)
        assert e.value.code == code, over
    with pytest.raises(abi.ZeroError) as e:                          # beyond the element limit
        abi.zero_cpu_adam_step(0x1000, 0x2000, 0x3000, 0x4000, "f16", abi.ZERO_MAX_ELEMS + 1, hp, 1.0, False,
                               0x5000, "f16", 1)
    assert e.value.code == abi.ZERO_EINVAL and "2^34" in str(e.value)
    bad = abi.adam_hparams(1e-3, 1.0, 0.999, 1e-8, 0.0, 1.0, 1)      # beta1 = 1
    with pytest.raises(abi.ZeroError):
        abi.zero_cpu_adam_step(t[0], t[1], t[2], g16, "f16", 64, bad, 1.0, False, out, "f16", 1)
    with pytest.raises(ValueError):                                   # buffers shorter than n
        abi.zero_cpu_adam_step(t[0], t[1], t[2], g16, "f16", 65, hp, 1.0, False, out, "f16", 1)
    with pytest.raises(abi.ZeroError):
        abi.zero_cpu_set_isa(abi.zero_cpu_isa() + 1)
