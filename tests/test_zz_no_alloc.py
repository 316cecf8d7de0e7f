"""zero_grad_norm_noalloc, the allocation-free norm, against zero_grad_norm.

The variant keeps its partial sums in a static device array instead of a
caller's workspace.  Through the C ABI, calls in a row on one GPU -- each
smaller than the one before, so the array holds a larger call's partials when
a smaller one starts -- must give the same norm, clip multiplier and flag as
zero_grad_norm with a workspace, bit for bit (same kernels, same summation
tree), and the norm must meet the parity bar against the oracle's exact norm.
"""

import numpy as np
import pytest
import torch

from oracle import rounding, step
from tolerance import coef_ok, norm_ok

pytestmark = pytest.mark.gpu

TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import abi as _abi
    return _abi


def _note(msg):
    print(msg, flush=True)


def _grad(n, dt, std, seed):
    rng = np.random.default_rng(seed)
    return rounding.narrow((rng.standard_normal(n) * std).astype(np.float32), dt)


def _outputs():
    return (torch.zeros(1, dtype=torch.int32, device="cuda"), torch.zeros(1, dtype=torch.float64, device="cuda"),
            torch.zeros(1, dtype=torch.float32, device="cuda"))


def _run_both(abi, bits, dt, inv_s, extra, max_norm):
    n = bits.size
    g = torch.from_numpy(bits.view(np.int16)).cuda().view(TORCH16[dt])
    d_extra = None if extra is None else torch.tensor(extra, dtype=torch.float64, device="cuda")
    n_extra = 0 if extra is None else len(extra)
    ws = torch.empty(abi.zero_workspace_bytes(n, 1), dtype=torch.uint8, device="cuda")
    f1, nrm1, c1 = _outputs()
    abi.zero_grad_norm(g, n, dt, inv_s, ws, 1, d_extra, n_extra, max_norm, f1, nrm1, c1)
    f2, nrm2, c2 = _outputs()
    abi.zero_grad_norm_noalloc(g, n, dt, inv_s, d_extra, n_extra, max_norm, f2, nrm2, c2)
    torch.cuda.synchronize()
    return (int(f1.item()), nrm1.item(), np.float32(c1.item())), (int(f2.item()), nrm2.item(), np.float32(c2.item()))


def test_noalloc_equals_the_workspace_norm_on_calls_in_a_row(abi):
    cases = [
        # n, dtype, std, inverse loss scale, extra sums of squares, max_norm
        (20_000_003, "bf16", 1e-3, 1.0, None, 1.0),              # two-stage fold (9766 partial sums)
        (300_001, "f16", 1e-3 * 16, 2.0 ** -4, [0.25, 1.5], 0.5),  # smaller: single stage, extra sums
        (4_099, "bf16", 1e-2, 1.0, None, 1.0),                   # smaller still: one partial sum and a tail
    ]
    for k, (n, dt, std, inv_s, extra, max_norm) in enumerate(cases):
        _note(f"noalloc call {k}: n={n} {dt} inv_s={inv_s} extra={extra}")
        bits = _grad(n, dt, std, 40 + k)
        ws_out, na_out = _run_both(abi, bits, dt, inv_s, extra, max_norm)
        assert na_out[0] == ws_out[0] == 0
        assert np.float64(na_out[1]).view(np.uint64) == np.float64(ws_out[1]).view(np.uint64), (na_out, ws_out)
        assert na_out[2].view(np.uint32) == ws_out[2].view(np.uint32), (na_out, ws_out)
        sumsq = step.sumsq_exact(bits, dt, inv_s) + sum(extra or [])
        ref = step.norm_from_sumsq(sumsq)
        norm_ok(na_out[1], ref, n, n_extra=len(extra or []))
        coef_ok(na_out[2], step.clip_coef(ref, max_norm))


def test_noalloc_flags_a_non_finite_gradient_like_the_workspace_norm(abi):
    bits = _grad(70_001, "f16", 1e-3, 9)
    bits[12_345] = np.uint16(0x7C00)                 # +inf
    ws_out, na_out = _run_both(abi, bits, "f16", 1.0, None, 1.0)
    assert ws_out[0] == na_out[0] == 1 | 2            # non-finite gradient, non-finite sum
    assert np.isinf(ws_out[1]) and np.isinf(na_out[1])
