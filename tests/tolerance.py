"""Parity tolerances for the AdamW outputs, derived once for every test.

The oracle computes the update in fp64 from the fp32 inputs and rounds once;
the kernels (and the host AdamW) compute it in fp32 operation by operation,
each operation adding at most u = 2^-24 relative error (round to nearest).
Following the operations of the update, the absolute error of each output is
bounded by a few u times the sum of the magnitudes of the terms that form it
(the standard bound for a short sum of products), not by its own magnitude:

* m' = b1*m + (1-b1)*g                 -> 4u (|b1 m| + |(1-b1) g|)
* v' = b2*v + (1-b2)*g^2               -> 8u (|b2 v| + |(1-b2) g^2|)
* p' = p - lr*(m^/(sqrt(v^)+eps) + wd*p)
                                       -> 24u (|p| + lr*A + lr*wd*|p|),
  A = (|b1 m| + |(1-b1) g|) / bc1 / (sqrt(v'/bc2) + eps)

where g = grad * inv_loss_scale * coef.  The p' bound matters where the
update nearly cancels p: the result is small but its error is a few ulps of
the operands.  Over several steps the kernels evolve their own state and the
oracle its own, so `AdamTrack` carries the differences forward through the
update (m and v scale by b1 and b2; p by 1 + lr*wd plus lr times the change of
m^/(sqrt(v^)+eps)) and adds each step's fresh bound.  The 16-bit parameter is
the round-to-nearest-even of the fp32 master: within one 16-bit ulp of the
oracle's, or within the master's bound plus one 16-bit rounding.

The global norm.  The oracle's is exact up to two roundings (the exact
rational sum of squares rounded to fp64, then a correctly rounded square
root): relative error <= 1.5 u64, u64 = 2^-53.  The kernels form each square
in fp64 (one rounding; the 16-bit value times a power of two is exact) and
add the squares along a fixed tree.  Every partial sum is a sum of
nonnegative terms, so the computed sum S' satisfies |S' - S| <= g(D+1) S with
g(k) = k u64 / (1 - k u64) and D the largest number of additions on any
path from a square to the root (the standard bound for recursive summation
of nonnegative terms, Higham, "Accuracy and Stability of Numerical
Algorithms", ch. 4).  The paths:
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

U32 = 2.0 ** -24
U64 = 2.0 ** -53
K_M, K_V, K_P = 4, 8, 24
ULP16_REL = {"f16": 2.0 ** -10, "bf16": 2.0 ** -7}
F16_MIN_ULP = 2.0 ** -24                 # fp16 subnormal spacing
FLOOR = 1e-38                            # below fp32's normal range: exact zeros compare equal


def _scalars(hp, step):
    b1, b2 = float(np.float32(hp.beta1)), float(np.float32(hp.beta2))
    return (b1, b2, 1.0 - b1 ** step, 1.0 - b2 ** step, float(np.float32(hp.lr)),
            float(np.float32(hp.weight_decay)), float(np.float32(hp.eps)))


def adam_bounds(master, m, v, grad_bits, grad_dtype, hp, step, coef):
    """Per-element absolute error bounds (p, m, v) of one fp32 AdamW update."""
    p = np.asarray(master, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    g = rounding.widen(grad_bits, grad_dtype).astype(np.float64) * float(hp.inv_loss_scale) * float(np.float32(coef))
    b1, b2, bc1, bc2, lr, wd, eps = _scalars(hp, step)
    m_terms = np.abs(b1 * m) + np.abs((1.0 - b1) * g)
    v_terms = np.abs(b2 * v) + np.abs((1.0 - b2) * g * g)
    denom = np.sqrt((b2 * v + (1.0 - b2) * g * g) / bc2) + eps
    a = m_terms / bc1 / denom
    p_terms = np.abs(p) + lr * a + lr * wd * np.abs(p)
    return K_P * U32 * p_terms + FLOOR, K_M * U32 * m_terms + FLOOR, K_V * U32 * v_terms + FLOOR


def within(got, ref, bound, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = np.flatnonzero(np.abs(got - ref) > bound)
    assert bad.size == 0, f"{what}: {bad.size} out of tolerance, first {bad[:3]}, got {got[bad[:3]]} " \
                          f"oracle {ref[bad[:3]]} bound {np.broadcast_to(bound, got.shape)[bad[:3]]}"


def adam_ok(got, ref, inputs, grad_bits, grad_dtype, hp, step, coef, param_dtype, what):
    """One update from the same inputs.  got / ref: (master, m, v, param_bits);
    inputs: the oracle's (master, m, v) before the update."""
    return AdamTrack().check(got, ref, inputs, grad_bits, grad_dtype, hp, step, coef, param_dtype, what)


class AdamTrack:
    """Bounds for a sequence of updates where each side evolves its own state."""

    def __init__(self):
        self.dp = self.dm = self.dv = 0.0

    def check(self, got, ref, inputs, grad_bits, grad_dtype, hp, step, coef, param_dtype, what):
        b1, b2, bc1, bc2, lr, wd, eps = _scalars(hp, step)
        fp, fm, fv = adam_bounds(*inputs, grad_bits, grad_dtype, hp, step, coef)
        cm, cv = b1 * self.dm, b2 * self.dv                 # carried into m', v'
        v_hat = np.asarray(ref[2], np.float64) / bc2
        m_hat = np.abs(np.asarray(ref[1], np.float64)) / bc1
        dv_hat = cv / bc2
        with np.errstate(divide="ignore", invalid="ignore"):
            d_sqrt = np.where(v_hat > 0, dv_hat / (2 * np.sqrt(v_hat)), np.inf)
        d_sqrt = np.minimum(d_sqrt, np.sqrt(dv_hat))
        denom = np.sqrt(v_hat) + eps
        d_ratio = 2 * (cm / bc1 / denom + m_hat * d_sqrt / (denom * denom))   # twice the first-order change
        bp = (1 + lr * wd) * self.dp + lr * d_ratio + fp
        bm, bv = cm + fm, cv + fv
        within(got[0], ref[0], bp, f"{what} master")
        within(got[1], ref[1], bm, f"{what} m")
        within(got[2], ref[2], bv, f"{what} v")
        param16_ok(got[3], ref[3], param_dtype, f"{what} param", master_bound=bp)
        self.dp, self.dm, self.dv = bp, bm, bv
        return bp


def param16_ok(got_bits, ref_bits, dtype, what, master_bound=0.0):
    d = np.abs(rounding.ordered16(got_bits) - rounding.ordered16(ref_bits))
    far = np.flatnonzero(d > 1)
    if far.size == 0:
        return
    g = rounding.widen(np.asarray(got_bits)[far], dtype).astype(np.float64)
    r = rounding.widen(np.asarray(ref_bits)[far], dtype).astype(np.float64)
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.maximum(mag * ULP16_REL[dtype], F16_MIN_ULP if dtype == "f16" else 0.0)
    bound = np.broadcast_to(master_bound, np.shape(got_bits))[far] + ulp
    bad = far[np.abs(g - r) > bound]
    assert bad.size == 0, f"{what}: {bad.size} params beyond one ulp and the master's bound, " \
                          f"e.g. got {rounding.widen(np.asarray(got_bits)[bad[:3]], dtype)} " \
                          f"oracle {rounding.widen(np.asarray(ref_bits)[bad[:3]], dtype)}"


def _ceil_div(a, b):
    return -(-a // b)


def norm_chain(n, n_extra=0):
    """D: the most fp64 additions between one square and the kernels' norm."""
    count = _ceil_div(int(n), 2048) + 1024
    chunk = max(4096, _ceil_div(count, 1024))
    fold = _ceil_div(chunk, 2048) + 1 + 3 + 6 + 4 if count > 8192 else 0
    return 33 + 6 + 4 + fold + 2 + 3 + 6 + 16 + int(n_extra)


def norm_rel(n, n_extra=0):
    """Relative bound on |kernel norm - oracle norm| for an n-element gradient."""
    d = norm_chain(n, n_extra)
    return ((d + 1) / 2 + 2.5) * U64 / (1 - (d + 1) * U64)


def norm_ok(got, ref, n, n_extra=0, what="norm"):
    got, ref = float(got), float(ref)
    bound = norm_rel(n, n_extra) * ref
    assert abs(got - ref) <= bound, f"{what}: {got!r} vs oracle {ref!r}, |diff| {abs(got - ref):.3g} > {bound:.3g}"


def coef_ok(got, ref, what="clip coefficient"):
    got, ref = np.float32(got), np.float32(ref)
    assert abs(float(got) - float(ref)) <= float(np.spacing(ref)), f"{what}: {got!r} vs oracle {ref!r}"
