"""Every emulated owner in one launch, and the device step count.

zero_reduce_owners must equal one zero_reduce_shard per owner (outputs and
partial sums, so the norm too) bit for bit, and zero_adam_step_owners one
zero_adam_step per owner, for strides that keep the vector path and strides
that do not.  The AdamW scalars come from a device table indexed by the
device step count: an index outside the table skips the update and says so
in the flag.  zero_step_end advances the count only for an applied step
(CMU 11-868 Lecture 18 notes §2.5: every rank emulated in one process).
Expected values come from the single-owner entry points, whose parity with
the oracle is covered in test_gpu_kernels.py, and from the oracle for AdamW.
"""

import ctypes

import numpy as np
import pytest
import torch

from oracle import rounding, step
from oracle.step import AdamHparams
from tolerance import adam_parity

pytestmark = pytest.mark.gpu

TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}
HP = AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, inv_loss_scale=2.0 ** -3)


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import abi as _abi
    return _abi


def _note(msg):
    print(msg, flush=True)


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _b32(t):
    return t.detach().view(torch.int32).cpu().numpy()


def _rand16(rng, n, std, dtype):
    return rounding.narrow((rng.standard_normal(n) * std).astype(np.float32), dtype)


def _to16(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(TORCH16[dtype])


def _state(abi, t, t0):
    st = abi.step_state(t, t0)
    return torch.frombuffer(bytearray(st), dtype=torch.int64).cuda()


def _counters(state):
    st = [int(x) for x in state.cpu()]
    return st[0], st[1], st[2], st[4] & 0xFFFFFFFF


def _table(abi, hp, t0, length):
    rows = b"".join(bytes(abi.zero_adam_consts_fill(
        abi.adam_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.inv_loss_scale, t)))
        for t in range(t0, t0 + length))
    return torch.frombuffer(bytearray(rows), dtype=torch.float32).cuda()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nd, owners, n, gap", [
    (4, 4, 262_147, 0),        # stride not a multiple of 4: the launch goes element by element
    (4, 4, 262_144, 0),        # stride a multiple of 4: the vector path for every owner
    (3, 2, 100_003, 5),        # gaps between owners' slices
    (16, 5, 4_099, 1),
    (8, 3, 1, 0),
    (100, 2, 5_000, 4),        # more than 64 ranks: the pointer table in the workspace, owner offsets on top
    (65, 3, 2_051, 3)])
def test_reduce_owners_equals_per_owner_calls(abi, dtype, nd, owners, n, gap):
    _note(f"reduce owners {dtype} nd={nd} owners={owners} n={n} gap={gap}")
    rng = np.random.default_rng(nd * 101 + owners * 7 + n)
    stride = n + gap
    span = (owners - 1) * stride + n
    local = [_to16(_rand16(rng, span, 1e-3, dtype), dtype) for _ in range(nd)]
    out = torch.full((owners, stride), 7, dtype=TORCH16[dtype], device="cuda")
    ws = torch.empty(abi.zero_workspace_bytes(n, owners), dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    abi.zero_reduce_owners(local, n, owners, stride, dtype, 1.0, out, stride, ws, flag)
    ref = torch.full((owners, stride), 7, dtype=TORCH16[dtype], device="cuda")
    ws_ref = torch.empty_like(ws)
    flag_ref = torch.zeros_like(flag)
    for o in range(owners):
        abi.zero_reduce_shard([x[o * stride:o * stride + n] for x in local], n, dtype, 1.0, ref[o, :n], ws_ref, o,
                              flag_ref)
    norms = []
    for w, f in ((ws, flag), (ws_ref, flag_ref)):
        nrm = torch.zeros(1, dtype=torch.float64, device="cuda")
        coef = torch.zeros(1, dtype=torch.float32, device="cuda")
        abi.zero_grad_norm(None, n, dtype, 1.0, w, owners, None, 0, 1.0, f, nrm, coef)
        norms.append((nrm.item(), coef.item()))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref))            # the gaps keep their 7s too
    assert int(flag.item()) == int(flag_ref.item()) == 0
    assert norms[0] == norms[1]
    # and against the oracle for one owner
    o = owners - 1
    expect, bad = step.reduce_shard([_bits(x[o * stride:o * stride + n]) for x in local], dtype)
    assert not bad and np.array_equal(_bits(out[o, :n]), expect)


@pytest.mark.parametrize("gdt, pdt", [("bf16", "bf16"), ("f16", "f16"), ("f16", "bf16")])
@pytest.mark.parametrize("owners, n, gap", [(4, 262_144, 0), (4, 262_147, 0), (3, 50_001, 3), (1, 77_777, 0)])
def test_adam_owners_equals_the_oracle_per_owner(abi, gdt, pdt, owners, n, gap):
    _note(f"adam owners {gdt}->{pdt} owners={owners} n={n} gap={gap}")
    rng = np.random.default_rng(owners * 13 + n)
    stride = n + gap
    size = owners * stride
    p = (rng.standard_normal(size) * 0.02).astype(np.float32)
    m = (rng.standard_normal(size) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(size) * 1e-8).astype(np.float32)
    g = _rand16(rng, size, 1e-4 / HP.inv_loss_scale, gdt)
    d = [torch.from_numpy(a.copy()).cuda() for a in (p, m, v)]
    dg = _to16(g, gdt)
    param = torch.zeros(size, dtype=TORCH16[pdt], device="cuda")
    coef = torch.tensor([0.75], dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    t0, t = 3, 5
    table = _table(abi, HP, t0, 4)
    state = _state(abi, t, t0)
    s = stride if owners > 1 else 0
    abi.zero_adam_step_owners(d[0], d[1], d[2], s, dg, gdt, s, n, owners, table, 4, state, coef, flag, param, s, pdt)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    got = [x.cpu().numpy() for x in d] + [_bits(param)]
    for o in range(owners):
        sl = slice(o * stride, o * stride + n)
        ref = step.adam_update(p[sl], m[sl], v[sl], g[sl], gdt, HP, t, np.float32(0.75), pdt)
        adam_parity(tuple(x[sl] for x in got), ref, pdt, f"owner {o}")
        if gap:
            gl = slice(o * stride + n, (o + 1) * stride)      # the gaps are untouched
            assert np.array_equal(got[0][gl], p[gl]) and not got[3][gl].any()


def test_adam_owners_outside_the_table_skips_and_flags(abi):
    n = 10_000
    p = torch.ones(n, device="cuda")
    m, v = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    g = torch.full((n,), 0.5, dtype=torch.bfloat16, device="cuda")
    param = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    coef = torch.ones(1, device="cuda")
    table = _table(abi, HP, 10, 2)
    for t in (9, 12, 100):                       # before the table, just past it, far past it
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        abi.zero_adam_step_owners(p, m, v, 0, g, "bf16", 0, n, 1, table, 2, _state(abi, t, 10), coef, flag, param,
                                  0, "bf16")
        torch.cuda.synchronize()
        assert int(flag.item()) == abi.ZERO_FLAG_NO_CONSTS, t
        assert torch.all(p == 1).item() and not param.any().item() and not m.any().item()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    abi.zero_adam_step_owners(p, m, v, 0, g, "bf16", 0, n, 1, table, 2, _state(abi, 11, 10), coef, flag, param, 0,
                              "bf16")
    torch.cuda.synchronize()
    assert int(flag.item()) == 0 and not torch.all(p == 1).item()


def test_step_end_advances_only_applied_steps(abi):
    assert ctypes.sizeof(abi.zero_step_state) == 40
    state = _state(abi, 7, 1)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    abi.zero_step_end(flag, state)                            # applied
    flag.fill_(abi.ZERO_FLAG_NONFINITE_GRAD | abi.ZERO_FLAG_NONFINITE_NORM)
    abi.zero_step_end(flag, state)                            # skipped
    torch.cuda.synchronize()
    assert _counters(state) == (8, 1, 1, 3) and int(flag.item()) == 0
    abi.zero_step_end(flag, state)
    torch.cuda.synchronize()
    assert _counters(state) == (9, 2, 1, 0)


def test_empty_owner_calls(abi):
    # n = 0: the reduce writes one zero partial sum per owner, AdamW nothing;
    # the norm then comes from the extra sums of squares alone; the step ends.
    owners = 3
    ws = torch.empty(abi.zero_workspace_bytes(0, owners), dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = torch.zeros(8, dtype=torch.float16, device="cuda")
    abi.zero_reduce_owners([t, t], 0, owners, 0, "f16", 1.0, t, 0, ws, flag)
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    coef = torch.zeros(1, dtype=torch.float32, device="cuda")
    extra = torch.tensor([9.0, 16.0], dtype=torch.float64, device="cuda")
    abi.zero_grad_norm(None, 0, "f16", 1.0, ws, owners, extra, 2, 1.0, flag, norm, coef)
    p = torch.ones(8, device="cuda")
    table = _table(abi, HP, 1, 1)
    state = _state(abi, 1, 1)
    abi.zero_adam_step_owners(p, p.clone(), p.clone(), 0, t, "f16", 0, 0, owners, table, 1, state, coef, flag, t, 0,
                              "f16")
    abi.zero_step_end(flag, state)
    torch.cuda.synchronize()
    assert norm.item() == 5.0 and coef.item() == np.float32(1.0 / (5.0 + 1e-6))
    assert _counters(state) == (2, 1, 0, 0) and torch.all(p == 1).item()
