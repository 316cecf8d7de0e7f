"""Pins for oracle.rounding: bf16 against torch's CPU cast (a library routine),
fp16 against hand-worked IEEE values, round trips over every 16-bit pattern."""

import numpy as np
import pytest
import torch

from oracle import rounding


def _patterns_bf16_neighbourhood():
    # Every upper half, with low halves at and around the rounding boundary
    # plus a few arbitrary ones: 2**16 * 10 fp32 patterns.
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000, 0x4000],
                    dtype=np.uint32)
    return (hi[:, None] | lows[None, :]).ravel()


def test_bf16_matches_torch_cast():
    u = _patterns_bf16_neighbourhood()
    x = u.view(np.float32)
    ours = rounding.narrow(x, "bf16")
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN (the payload is not compared).
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x007F) != 0)


def test_bf16_random_patterns_match_torch():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    ours = rounding.narrow(x, "bf16")
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ok = ~np.isnan(x)
    assert np.array_equal(ours[ok], ref[ok])


@pytest.mark.parametrize("value, bits", [
    (65504.0, 0x7BFF),                 # largest finite fp16
    (65519.996, 0x7BFF),               # below the halfway point to 2**16
    (65520.0, 0x7C00),                 # halfway: ties to even -> inf
    (2.0 ** -24, 0x0001),              # smallest subnormal
    (2.0 ** -25, 0x0000),              # halfway to zero: ties to even -> 0
    (1.5 * 2.0 ** -24, 0x0002),        # halfway between 1 and 2 ulps -> even (2)
    (1.0 + 2.0 ** -11, 0x3C00),        # halfway above 1.0 -> even (1.0)
    (1.0 + 3 * 2.0 ** -11, 0x3C02),    # halfway between 0x3C01 and 0x3C02 -> even
    (-2.0 ** -14, 0x8400),             # smallest negative normal
    (2.0 ** -14 - 2.0 ** -24, 0x03FF), # largest subnormal
])
def test_fp16_hand_worked(value, bits):
    assert int(rounding.narrow(np.array([value], np.float32), "f16")[0]) == bits


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_pattern_round_trips(dtype):
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = rounding.is_finite16(b, dtype)
    x = rounding.widen(b, dtype)
    back = rounding.narrow(x, dtype)
    assert np.array_equal(back[fin], b[fin])
    # Infinities round-trip too; NaN stays NaN.
    inf = ~fin & np.isinf(x)
    assert np.array_equal(back[inf], b[inf])
    assert np.all(np.isnan(rounding.widen(back[np.isnan(x)], dtype)))


def test_widen_is_exact_against_float64_definition():
    # bf16 is the upper half of an fp32 pattern; fp16 per IEEE binary16.
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    val = np.where(e == 0, sign * f * 2.0 ** -24, sign * (1 + f / 1024) * 2.0 ** (e.astype(np.float64) - 15))
    ok = e != 31
    with np.errstate(invalid="ignore"):                 # the NaN patterns, masked out below
        wide = rounding.widen(b, "f16").astype(np.float64)
    assert np.array_equal(wide[ok], val[ok])


def test_ordered16():
    b = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3C00, 0x3C01], np.uint16)
    o = rounding.ordered16(b)
    assert list(o) == [0, 0, 1, -1, 0x3C00, 0x3C01]
