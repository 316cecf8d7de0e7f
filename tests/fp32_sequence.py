"""The fp32 operation sequence that the library's AdamW evaluates, in numpy.

This is not the oracle.  The oracle defines the update in fp64 and rounds once
(ZeRO paper, section 3 and its mixed-precision Adam; Loshchilov and Hutter's
decoupled weight decay).  The device kernel and the host AdamW instead
evaluate it one fp32 operation at a time, in a documented order, each
operation rounded to nearest, with no fused multiply-add and with correctly
rounded division and square root.  This module writes that order out so that
tests can check, bit for bit, that both evaluate exactly it; how far the
sequence may stray from the oracle's result is bounded separately by
`tolerance.py`.  numpy evaluates each float32 ufunc with one IEEE rounding.

Order, for g16 the 16-bit gradient:
    g     = widen(g16) * (inv_loss_scale * coef)
    m'    = b1*m + (1-b1)*g
    v'    = b2*v + (1-b2)*(g*g)
    denom = sqrt(v' * inv_bc2) + eps
    p'    = p - lr*((m' * inv_bc1) / denom + wd*p)
    p16   = round_to_nearest_even_16(p')
with 1-b1, 1-b2 formed in fp64 and rounded to fp32, bc_k = fp32(1 - b_k^t)
from fp64, inv_bc_k = fp32(1 / bc_k) from fp64.
"""

import numpy as np

from oracle import rounding

F32 = np.float32


def consts(hp, step, coef):
    """The fp32 scalars of one step (keys follow the library's zero_adam_consts)."""
    b1, b2 = F32(hp.beta1), F32(hp.beta2)
    bc1 = F32(1.0 - float(b1) ** int(step))
    bc2 = F32(1.0 - float(b2) ** int(step))
    return {
        "lr": F32(hp.lr), "beta1": b1, "beta2": b2,
        "one_minus_beta1": F32(1.0 - float(b1)), "one_minus_beta2": F32(1.0 - float(b2)),
        "eps": F32(hp.eps), "weight_decay": F32(hp.weight_decay),
        "inv_loss_scale": F32(hp.inv_loss_scale),
        "inv_bias_corr1": F32(1.0 / float(bc1)), "inv_bias_corr2": F32(1.0 / float(bc2)),
        "grad_scale": F32(hp.inv_loss_scale) * F32(coef),
    }


def adamw(master, m, v, grad_bits, grad_dtype, hp, step, coef, param_dtype):
    """One update; returns (master', m', v', param16 bits)."""
    c = consts(hp, step, coef)
    p = np.asarray(master, F32)
    m = np.asarray(m, F32)
    v = np.asarray(v, F32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore", divide="ignore"):
        g = rounding.widen(grad_bits, grad_dtype) * c["grad_scale"]
        m2 = c["beta1"] * m + c["one_minus_beta1"] * g
        v2 = c["beta2"] * v + c["one_minus_beta2"] * (g * g)
        denom = np.sqrt(v2 * c["inv_bias_corr2"]) + c["eps"]
        p2 = p - c["lr"] * ((m2 * c["inv_bias_corr1"]) / denom + c["weight_decay"] * p)
    for a in (g, m2, v2, denom, p2):
        assert a.dtype == F32
    return p2, m2, v2, rounding.narrow(p2, param_dtype)


def edge_inputs(n, grad_dtype, inv_loss_scale, seed):
    """Seeded (grad16 bits, master, m, v) in the usual recipe (gradient std 1e-3
    before loss scaling, parameters std 0.02, m std 1e-4, v = |std 1e-6|) with
    one kind of edge value per eighth of the range: zero gradients; zero m and
    v; fp32-subnormal v; 16-bit subnormal gradients; the largest finite
    gradients (g*g overflows for bf16); zero parameters; fp32-subnormal m."""
    rng = np.random.default_rng(seed)
    g = rounding.narrow((rng.standard_normal(n) * 1e-3 / inv_loss_scale).astype(F32), grad_dtype)
    p = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(F32)
    k = n // 8
    sign = lambda: (rng.integers(0, 2, k) << 15).astype(np.uint16)
    g[:k] = 0
    m[k:2 * k] = 0
    v[k:2 * k] = 0
    v[2 * k:3 * k] = F32(1e-40)
    g[3 * k:4 * k] = rng.integers(1, 0x400 if grad_dtype == "f16" else 0x80, k).astype(np.uint16) | sign()
    g[4 * k:5 * k] = np.uint16(0x7BFF if grad_dtype == "f16" else 0x7F7F) | sign()
    p[5 * k:6 * k] = 0
    m[6 * k:7 * k] = F32(-3e-42)
    return g, p, m, v


def same_bits(got, ref, what):
    """Assert equal fp32 (or 16-bit) patterns; reports the first differences."""
    got = np.ascontiguousarray(got)
    ref = np.ascontiguousarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    view = np.uint32 if got.dtype.itemsize == 4 else np.uint16
    gb, rb = got.view(view), ref.view(view)
    bad = np.flatnonzero(gb != rb)
    assert bad.size == 0, f"{what}: {bad.size} of {gb.size} differ, first at {bad[:4]}: " \
                          f"got {got[bad[:4]]} expected {ref[bad[:4]]}"
