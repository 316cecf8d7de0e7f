"""Seeded AdamW inputs with edge values mixed in, for the parity tests.

Input generation only: no part of the update is computed here.
"""

import numpy as np

from oracle import rounding

F32 = np.float32


def edge_inputs(n, grad_dtype, inv_loss_scale, seed):
    """Seeded (grad16 bits, master, m, v) in the usual recipe (gradient std 1e-3
    before loss scaling, parameters std 0.02, m std 1e-4, v = |std 1e-6|) with
    one kind of edge value per eighth of the range: zero gradients; zero m and
    v; fp32-subnormal v; 16-bit subnormal gradients; the largest finite
    gradients (for bf16, v' then overflows fp32); zero parameters;
    fp32-subnormal m."""
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
