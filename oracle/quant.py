"""Block-quantised 16-bit parameters for the gather (ZeRO++ quantised weights).

Test infrastructure: see the package docstring.

Pages: ZeRO++ sends the ZeRO-3 parameter all-gather in low precision, and
quantises in blocks because one scale per tensor lets a few large values
stretch the scale so the rest round coarsely; the notes quantise 1M weights
with 64 values 20 times larger and report INT8 11.25% (per tensor) vs 0.89%
(one scale per 256) and INT4 98.69% vs 14.53% (CMU 11-868 Lecture 18 notes
§4.5; exercise 10).

Readings (the pages give no formula):
* symmetric absmax quantisation: scale = max|x| / qmax over each block of
  256 consecutive elements (the last block may be shorter), qmax = 127 for
  INT8 and 7 for INT4; code = clamp(round(x / scale), -qmax, qmax) with
  round-half-to-even; a block of zeros has scale 0 and codes 0;
* the arithmetic is float32: x is the float32 value of the 16-bit input, the
  scale is an IEEE float32 division, x / scale is an IEEE float32 division;
* dequantised value = round-to-nearest-even into 16 bits of float32(code *
  scale);
* INT4 codes are two's complement nibbles, two per byte, the even element
  in the low nibble;
* the error figure on the page is the relative L2 error ||x' - x|| / ||x||
  with x ~ N(0, 1) and 64 elements multiplied by 20 (the reading under which
  the printed figures come out; see the tests).
"""

import numpy as np

from .rounding import narrow, widen

BLOCK = 256
QMAX = {8: 127, 4: 7}


def _qmax(bits):
    if bits not in QMAX:
        raise ValueError("bits must be 8 or 4")
    return QMAX[bits]


def block_scales(x32, bits, block=BLOCK):
    """float32 absmax / qmax per block of a float32 vector."""
    qmax = np.float32(_qmax(bits))
    n = x32.shape[0]
    nb = -(-n // block)
    padded = np.zeros(nb * block, np.float32)
    padded[:n] = np.abs(x32)
    return (padded.reshape(nb, block).max(axis=1) / qmax).astype(np.float32)


def quantize(bits16, dtype, bits, block=BLOCK):
    """16-bit patterns -> (int8 codes, one per element, and float32 scales)."""
    x = widen(bits16, dtype)
    scales = block_scales(x, bits, block)
    qmax = _qmax(bits)
    per_elem = np.repeat(scales, block)[:x.shape[0]]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(per_elem > 0, x / np.where(per_elem > 0, per_elem, np.float32(1)), np.float32(0))
    codes = np.clip(np.rint(ratio.astype(np.float32)), -qmax, qmax).astype(np.int8)
    return codes, scales


def dequantize(codes, scales, dtype, block=BLOCK):
    """(int8 codes, float32 scales) -> 16-bit patterns."""
    codes = np.asarray(codes, np.int8)
    per_elem = np.repeat(np.asarray(scales, np.float32), block)[:codes.shape[0]]
    return narrow(codes.astype(np.float32) * per_elem, dtype)


def pack4(codes):
    """INT4 codes (int8 in [-7, 7]) -> bytes, element 2i in the low nibble."""
    codes = np.asarray(codes, np.int8)
    if codes.shape[0] % 2:
        codes = np.concatenate([codes, np.zeros(1, np.int8)])
    nib = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def unpack4(packed, n):
    """Bytes -> INT4 codes as int8 (sign-extended nibbles), first n of them."""
    packed = np.asarray(packed, np.uint8)
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    both = np.empty(packed.shape[0] * 2, np.int8)
    both[0::2], both[1::2] = lo, hi
    both = np.where(both > 7, both - 16, both).astype(np.int8)
    return both[:n]


def relative_error(x, x_hat):
    """||x_hat - x||_2 / ||x||_2 in float64."""
    x = np.asarray(x, np.float64)
    return float(np.linalg.norm(np.asarray(x_hat, np.float64) - x) / np.linalg.norm(x))
