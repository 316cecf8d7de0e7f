"""The derived 16-bit parameter tolerance accepts what the fp32 master's
tolerance allows and nothing more: two ulps apart at ordinary magnitudes
fails; near zero, a difference within the master's absolute tolerance
passes even when it spans several 16-bit ulps."""

import numpy as np
import pytest

from oracle import rounding
from tolerance import param16_ok


def _b(vals, dt):
    return rounding.narrow(np.asarray(vals, np.float32), dt)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_one_ulp_passes_two_fail_at_ordinary_magnitude(dt):
    x = _b([0.02, -0.013, 1.5], dt)
    param16_ok(x, x, dt, "equal")
    param16_ok(x + np.uint16(1), x, dt, "one ulp")
    with pytest.raises(AssertionError):
        param16_ok(x + np.uint16(2), x, dt, "two ulps")


def test_near_zero_within_the_master_tolerance():
    # bf16 values of 3e-10 and 1e-10 differ by many ulps but by 2e-10 < 1e-9
    got, ref = _b([3e-10], "bf16"), _b([1e-10], "bf16")
    param16_ok(got, ref, "bf16", "cancellation")
    with pytest.raises(AssertionError):
        param16_ok(_b([3e-9], "bf16"), ref, "bf16", "beyond the absolute tolerance")
    # across zero in fp16: -0 against the smallest subnormal is one ulp in value
    # (two encodings apart) and passes; -1 against +1 subnormal is two and fails
    param16_ok(np.uint16([0x8000]), np.uint16([0x0001]), "f16", "-0 vs the smallest subnormal")
    with pytest.raises(AssertionError):
        param16_ok(np.uint16([0x8001]), np.uint16([0x0001]), "f16", "opposite subnormals")
