"""Parity tolerances for the AdamW outputs, derived once for every test.

The oracle computes the update in fp64 and rounds once; the kernels (and the
host AdamW) compute it in fp32 operation by operation.  Against it:

* master, m and v: |got - oracle| <= 1e-9 + 1e-6 |oracle|.  Each fp32
  operation adds at most half an ulp (2^-24 relative) and the update takes
  about ten of them; the absolute term covers values whose fp32 rounding is
  below 1e-9 (m and v of tiny gradients, and a master that the update brings
  close to zero, where p - lr*update cancels and the error of the operands,
  about one ulp of p, remains).
* the 16-bit parameter is the round-to-nearest-even of the fp32 master, so
  it may differ from the oracle's by one 16-bit ulp, or, where the master
  itself differs by up to the tolerance above (near zero, after
  cancellation), by that difference plus one 16-bit rounding.
"""

import numpy as np

from oracle import rounding

ABS_TOL = 1e-9
REL_TOL = 1e-6
ULP16_REL = {"f16": 2.0 ** -10, "bf16": 2.0 ** -7}
F16_MIN_ULP = 2.0 ** -24                 # fp16 subnormal spacing; bf16's is below any tolerance here


def state_ok(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = np.flatnonzero(np.abs(got - ref) > ABS_TOL + REL_TOL * np.abs(ref))
    assert bad.size == 0, f"{what}: {bad.size} out of tolerance, first {bad[:3]}, " \
                          f"got {got[bad[:3]]} oracle {ref[bad[:3]]}"


def param16_ok(got_bits, ref_bits, dtype, what):
    d = np.abs(rounding.ordered16(got_bits) - rounding.ordered16(ref_bits))
    far = np.flatnonzero(d > 1)
    if far.size == 0:
        return
    g = rounding.widen(np.asarray(got_bits)[far], dtype).astype(np.float64)
    r = rounding.widen(np.asarray(ref_bits)[far], dtype).astype(np.float64)
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.maximum(mag * ULP16_REL[dtype], F16_MIN_ULP if dtype == "f16" else 0.0)
    bound = ABS_TOL + REL_TOL * np.abs(r) + ulp
    bad = far[np.abs(g - r) > bound]
    assert bad.size == 0, f"{what}: {bad.size} params beyond one ulp and the master's tolerance, " \
                          f"e.g. got {rounding.widen(np.asarray(got_bits)[bad[:3]], dtype)} " \
                          f"oracle {rounding.widen(np.asarray(ref_bits)[bad[:3]], dtype)}"
