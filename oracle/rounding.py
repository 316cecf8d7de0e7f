"""fp32 <-> 16-bit conversions used by the oracle.

Test infrastructure: see the package docstring.

The pages keep parameters and gradients in fp16 (or bf16) and the optimizer
state in fp32, and copy the updated fp32 master back to the 16-bit parameter
(CMU 11-868 Lecture 18 notes §1.2 and §2.2 step 4; L3.2 Memory optimisation and
ZeRO §2.1).  They do not name a rounding mode; IEEE round-to-nearest-even with
gradual underflow is the reading taken here.

* fp16: ``numpy``'s float32 -> float16 cast, a library routine that rounds to
  nearest even and keeps subnormals.
* bf16: written out from the definition -- bf16 is the top 16 bits of the fp32
  pattern; rounding to nearest even adds 0x7FFF plus the lowest kept bit before
  the shift.  NaN maps to the quiet NaN 0x7FC0.

Pages cited by short name:
  L3.2  "L3.2 显存优化与 ZeRO" (yulong.wang)
"""

import numpy as np

DTYPES = ("f16", "bf16")


def _check(dtype):
    if dtype not in DTYPES:
        raise ValueError(f"16-bit dtype must be one of {DTYPES}, got {dtype!r}")


def widen(bits, dtype):
    """16-bit patterns (uint16) -> exact float32 values."""
    _check(dtype)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lowest_kept = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lowest_kept) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    rounded = np.where(is_nan, np.uint64(0x7FC0), rounded)
    return rounded.astype(np.uint16)


def narrow(x, dtype):
    """float32 values -> 16-bit patterns, round to nearest even."""
    _check(dtype)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        with np.errstate(over="ignore"):       # beyond the fp16 range rounds to infinity (IEEE)
            return x.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(x)


def is_finite16(bits, dtype):
    """True where the 16-bit pattern is a finite number (exponent field not all ones)."""
    _check(dtype)
    bits = np.asarray(bits, dtype=np.uint16)
    exp_mask = np.uint16(0x7C00) if dtype == "f16" else np.uint16(0x7F80)
    return (bits & exp_mask) != exp_mask


def ordered16(bits):
    """Map sign-magnitude 16-bit patterns to integers whose order is the numeric order.

    Used to measure distances in units in the last place (ulp): the distance
    between two finite values of the same 16-bit format is the difference of
    their ordered integers.  +0 and -0 both map to 0.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)
