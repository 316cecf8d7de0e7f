"""Parity bars for the AdamW outputs, the global norm and the clip multiplier.

The bar every parity test asserts (the sharded update must give the plain
data-parallel result, CMU 11-868 Lecture 18 notes §2.5):

* master, m, v:  |gpu - oracle| <= 1e-9 + 1e-6 * |oracle|, element by element;
* the 16-bit parameter: at most one ulp from the oracle's (the distance
  between the sign-magnitude patterns mapped to ordered integers, so +0 and
  -0 are the same point);
* the norm: relative 1e-5.

The library evaluates the AdamW update in fp64 in the oracle's own order,
with correctly rounded division and square root, and rounds each output to
fp32 once, so given the same clip multiplier its outputs equal the oracle's
bit for bit.  `adam_same` checks that stronger property; the parity tests
assert it wherever the device's clip multiplier equals the oracle's.

The norm also meets a derived bound far below 1e-5.  The oracle's norm is
exact up to two roundings (the exact rational sum of squares rounded to fp64,
then a correctly rounded square root): relative error <= 1.5 u64,
u64 = 2^-53.  The kernels form each square in fp64 (one rounding; the 16-bit
value times a power of two is exact) and add the squares along a fixed tree.
Every partial sum is a sum of nonnegative terms, so the computed sum S'
satisfies |S' - S| <= g(D+1) S with g(k) = k u64 / (1 - k u64) and D the
largest number of additions on any path from a square to the root (the
standard bound for recursive summation of nonnegative terms, Higham,
"Accuracy and Stability of Numerical Algorithms", ch. 4).  The paths:
  per lane           <= 33  (32 squares of a sum-of-squares range + 1 tail
                             element; 8 in the reduce)
  wave butterfly        6
  block's waves      <= 4
  fold, count > 8192  ceil(chunk / 2048) + 1, then 3 + 6 + 4
                      (chunk <= max(4096, ceil(count / 1024)))
  finalize            2 + 3 + 6 + 16, plus one per extra sum of squares
where count, the number of 2048-element partial sums, is at most
ceil(n / 2048) + 1024 (one short range per reduce call, at most 1024 calls).
The square root halves the relative error and adds one rounding, so the
norms differ by at most ((D + 1) / 2 + 2.5) u64 relative: about 5e-15 at
1.1e10 elements.  The clip coefficient is one fp32 rounding of nearly equal
fp64 quotients, so it is within one fp32 ulp of the oracle's.
"""

import numpy as np

from oracle import rounding

U64 = 2.0 ** -53
ADAM_ABS = 1e-9
ADAM_REL = 1e-6
NORM_REL = 1e-5


def _same_class(got, ref):
    """Positions where both are the same infinity or both are NaN."""
    both_nan = np.isnan(got) & np.isnan(ref)
    same_inf = np.isinf(got) & (got == ref)
    return both_nan | same_inf


def within(got, ref, what, abs_tol=ADAM_ABS, rel_tol=ADAM_REL):
    """|got - ref| <= abs_tol + rel_tol * |ref| element by element (fp32 arrays);
    an infinite or NaN oracle value must be matched by the same class."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    with np.errstate(invalid="ignore", over="ignore"):
        ok = np.isfinite(ref) & (np.abs(got - ref) <= abs_tol + rel_tol * np.abs(ref))
    bad = np.flatnonzero(~(ok | _same_class(got, ref)))
    assert bad.size == 0, f"{what}: {bad.size} of {got.size} beyond {abs_tol:g} + {rel_tol:g}*|oracle|, " \
                          f"first at {bad[:3]}: got {got[bad[:3]]} oracle {ref[bad[:3]]}"


def param16_ok(got_bits, ref_bits, dtype, what):
    """16-bit parameters at most one ulp apart."""
    got_bits = np.asarray(got_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    assert got_bits.shape == ref_bits.shape, f"{what}: shape {got_bits.shape} != {ref_bits.shape}"
    d = np.abs(rounding.ordered16(got_bits) - rounding.ordered16(ref_bits))
    nan = ~rounding.is_finite16(got_bits, dtype) & ~rounding.is_finite16(ref_bits, dtype)
    bad = np.flatnonzero((d > 1) & ~nan)
    assert bad.size == 0, f"{what}: {bad.size} params more than one ulp from the oracle, first at {bad[:3]}: " \
                          f"got {rounding.widen(got_bits[bad[:3]], dtype)} " \
                          f"oracle {rounding.widen(ref_bits[bad[:3]], dtype)}"


def adam_ok(got, ref, param_dtype, what):
    """The bar: got / ref are (master, m, v, param_bits) after the same update."""
    for a, b, name in zip(got[:3], ref[:3], ("master", "m", "v")):
        within(a, b, f"{what} {name}")
    param16_ok(got[3], ref[3], param_dtype, f"{what} param")


def same_bits(got, ref, what):
    """Assert equal fp32 (or 16-bit) patterns; reports the first differences."""
    got = np.ascontiguousarray(got)
    ref = np.ascontiguousarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert got.dtype.itemsize == ref.dtype.itemsize, f"{what}: dtype {got.dtype} != {ref.dtype}"
    view = np.uint32 if got.dtype.itemsize == 4 else np.uint16
    gb, rb = got.view(view), ref.view(view)
    bad = np.flatnonzero(gb != rb)
    assert bad.size == 0, f"{what}: {bad.size} of {gb.size} differ, first at {bad[:4]}: " \
                          f"got {got[bad[:4]]} expected {ref[bad[:4]]}"


def adam_same(got, ref, what):
    """Bit-identical (master, m, v, param_bits)."""
    for a, b, name in zip(got, ref, ("master", "m", "v", "param")):
        same_bits(a, b, f"{what} {name}")


def adam_parity(got, ref, param_dtype, what, same=True):
    """The bar, then (if `same`: both sides used the same clip multiplier) bit identity."""
    adam_ok(got, ref, param_dtype, what)
    if same:
        adam_same(got, ref, what)


def _ceil_div(a, b):
    return -(-a // b)


def norm_chain(n, n_extra=0):
    """D: the most fp64 additions between one square and the kernels' norm."""
    count = _ceil_div(int(n), 2048) + 1024
    chunk = max(4096, _ceil_div(count, 1024))
    fold = _ceil_div(chunk, 2048) + 1 + 3 + 6 + 4 if count > 8192 else 0
    return 33 + 6 + 4 + fold + 2 + 3 + 6 + 16 + int(n_extra)


def norm_rel(n, n_extra=0):
    """Derived relative bound on |kernel norm - oracle norm| for an n-element gradient."""
    d = norm_chain(n, n_extra)
    return ((d + 1) / 2 + 2.5) * U64 / (1 - (d + 1) * U64)


def norm_ok(got, ref, n, n_extra=0, what="norm"):
    """The bar (relative 1e-5), then the derived bound."""
    got, ref = float(got), float(ref)
    assert abs(got - ref) <= NORM_REL * abs(ref), f"{what}: {got!r} vs oracle {ref!r} beyond relative 1e-5"
    bound = norm_rel(n, n_extra) * ref
    assert abs(got - ref) <= bound, f"{what}: {got!r} vs oracle {ref!r}, |diff| {abs(got - ref):.3g} > {bound:.3g}"


def coef_ok(got, ref, what="clip coefficient"):
    got, ref = np.float32(got), np.float32(ref)
    assert abs(float(got) - float(ref)) <= float(np.spacing(ref)), f"{what}: {got!r} vs oracle {ref!r}"
