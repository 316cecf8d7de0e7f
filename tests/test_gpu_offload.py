"""GPU parity of the ZeRO-Offload update (``zero_offload_adam_step``).

The reduced gradient and the clip multiplier live on the GPU, the fp32 state
in host memory; the host state and the 16-bit parameters that come back to
the device are compared with the oracle's AdamW (the bar, and bit for bit),
and bit for bit with the host
AdamW called directly on the same inputs (the chunking and the overlap of
copies with the update change nothing) and with the GPU kernel keeping the
state in HBM.  Staging buffers down to the minimum
force many chunks and a ragged last one.
"""

import numpy as np
import pytest
import torch

from oracle import rounding, step
from oracle.step import AdamHparams
from zero_sharded_mixed_flat_amd import synth
from tolerance import adam_parity

pytestmark = pytest.mark.gpu

TORCH16 = synth.TORCH_DTYPES
HP = AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, inv_loss_scale=2.0 ** -4)


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import abi as _abi
    return _abi


def _note(msg):
    print(msg, flush=True)


def _abi_hp(abi, hp, t):
    return abi.adam_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.inv_loss_scale, t)


def _inputs(n, gdt, seed):
    rng = np.random.default_rng(seed)
    g = rounding.narrow((rng.standard_normal(n) * 1e-3 / HP.inv_loss_scale).astype(np.float32), gdt)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    return g, p, m, v


def _offload(abi, g, p, m, v, gdt, pdt, t, coef, flag, staging_bytes, threads=4, declared=None):
    n = g.size
    hm, hmm, hv = (torch.from_numpy(a.copy()) for a in (p, m, v))
    dg = torch.from_numpy(g.view(np.int16).copy()).cuda()
    dp = torch.full((n,), 7, dtype=torch.int16, device="cuda")
    dcoef = torch.tensor([coef], dtype=torch.float32, device="cuda")
    dflag = torch.tensor([flag], dtype=torch.int32, device="cuda")
    staging = torch.empty(staging_bytes, dtype=torch.uint8, pin_memory=True)
    abi.zero_offload_adam_step(hm, hmm, hv, dg, gdt, n, _abi_hp(abi, HP, t), dcoef, dflag, dp, pdt, staging,
                               threads, staging_bytes=declared)
    return hm.numpy(), hmm.numpy(), hv.numpy(), dp.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("gdt, pdt", [("bf16", "bf16"), ("f16", "f16"), ("f16", "bf16")])
@pytest.mark.parametrize("n", [1, 63, 64, 1000, 100_003])
@pytest.mark.parametrize("staging", [576, 64 + 8 * 4096, 64 + 8 * (1 << 20)])
def test_offload_matches_oracle_and_host_adam(abi, gdt, pdt, n, staging):
    _note(f"offload n={n} staging={staging} {gdt}->{pdt}")
    g, p, m, v = _inputs(n, gdt, n + staging)
    coef = np.float32(0.6)
    got = _offload(abi, g, p, m, v, gdt, pdt, 3, float(coef), 0, staging)
    ref = step.adam_update(p, m, v, g, gdt, HP, 3, coef, pdt)
    adam_parity(got, ref, pdt, "offload")
    # the same update by the host AdamW called directly: identical bits
    hm, hmm, hv = (torch.from_numpy(a.copy()) for a in (p, m, v))
    out = torch.zeros(n, dtype=torch.int16)
    abi.zero_cpu_adam_step(hm, hmm, hv, torch.from_numpy(g.view(np.int16).copy()), gdt, n, _abi_hp(abi, HP, 3),
                           float(coef), False, out, pdt, 2)
    for a, b in zip(got, (hm.numpy(), hmm.numpy(), hv.numpy(), out.numpy().view(np.uint16))):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)
    # and by the GPU kernel with the state kept in HBM: the offloaded step gives the same bits
    dm, dmm, dv = (torch.from_numpy(a.copy()).cuda() for a in (p, m, v))
    dpar = torch.zeros(n, dtype=torch.int16, device="cuda")
    abi.zero_adam_step(dm, dmm, dv, torch.from_numpy(g.view(np.int16).copy()).cuda(), gdt, n, _abi_hp(abi, HP, 3),
                       torch.tensor([coef], dtype=torch.float32, device="cuda"),
                       torch.zeros(1, dtype=torch.int32, device="cuda"), dpar, pdt)
    torch.cuda.synchronize()
    for a, b in zip(got, (dm.cpu().numpy(), dmm.cpu().numpy(), dv.cpu().numpy(),
                          dpar.cpu().numpy().view(np.uint16))):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)


def test_offload_skip_moves_nothing(abi):
    g, p, m, v = _inputs(5000, "bf16", 1)
    got = _offload(abi, g, p, m, v, "bf16", "bf16", 1, 1.0, 1, 64 + 8 * 1024)
    assert np.array_equal(got[0], p) and np.array_equal(got[1], m) and np.array_equal(got[2], v)
    assert np.all(got[3] == 7)                    # the device parameters keep their old values


def test_offload_rejects(abi):
    g, p, m, v = _inputs(100, "bf16", 2)
    with pytest.raises(ValueError):               # the binding refuses a staging tensor below the minimum
        _offload(abi, g, p, m, v, "bf16", "bf16", 1, 1.0, 0, 512)
    with pytest.raises(abi.ZeroError) as e:       # and so does the library, for a declared size below it
        _offload(abi, g, p, m, v, "bf16", "bf16", 1, 1.0, 0, 576, declared=512)
    assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError) as e:       # a clip multiplier of zero on the device
        _offload(abi, g, p, m, v, "bf16", "bf16", 1, 0.0, 0, 576)
    assert e.value.code == abi.ZERO_EINVAL and "clip multiplier" in str(e.value)
    got = _offload(abi, g, p, m, v, "bf16", "bf16", 1, 1.0, 0, 576)     # and the next call works
    assert not np.array_equal(got[0], p)


# ---------------------------------------------------------------------------
# the one-step-delayed update (zero_offload_begin / zero_offload_end)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gdt, pdt", [("bf16", "bf16"), ("f16", "f16")])
@pytest.mark.parametrize("n, threads", [(100_003, 4), (64, 16), (1, 1)])
def test_delayed_updates_equal_the_oracle_sequence(abi, gdt, pdt, n, threads):
    # Three steps through begin/end; each update is the oracle's from the
    # previous state, bit for bit, and the device parameters of step t reach
    # the device only when step t ends (one step late).
    _note(f"delayed offload {gdt}->{pdt} n={n} threads={threads}")
    rng = np.random.default_rng(n + threads)
    h = abi.Offload(threads)
    dbuf = torch.empty(2 * n, dtype=torch.int16, device="cuda")
    staging = torch.empty(64 + 8 * 4096, dtype=torch.uint8, pin_memory=True)     # several chunks at n = 100003
    _, p, m, v = _inputs(n, gdt, 77)
    hm, hmm, hv = (torch.from_numpy(a.copy()) for a in (p, m, v))
    dparam = torch.full((n,), 5, dtype=torch.int16, device="cuda")
    state = (p, m, v)
    prev_bits = np.full(n, 5, np.uint16)
    for t in range(1, 4):
        g = rounding.narrow((rng.standard_normal(n) * 1e-3 / HP.inv_loss_scale).astype(np.float32), gdt)
        coef = np.float32(0.5 + 0.1 * t)
        dg = torch.from_numpy(g.view(np.int16).copy()).cuda()
        dcoef = torch.tensor([coef], dtype=torch.float32, device="cuda")
        dflag = torch.zeros(1, dtype=torch.int32, device="cuda")
        h.begin(hm, hmm, hv, dg, gdt, n, _abi_hp(abi, HP, t), dcoef, dflag, pdt, dbuf, staging)
        dg.fill_(0)                               # the device may reuse the gradient buffer at once
        assert np.array_equal(dparam.cpu().numpy().view(np.uint16), prev_bits)   # still the last step's
        assert h.end(dparam) is True
        ref = step.adam_update(*state, g, gdt, HP, t, coef, pdt)
        got = (hm.numpy(), hmm.numpy(), hv.numpy(), dparam.cpu().numpy().view(np.uint16))
        adam_parity(got, ref, pdt, f"delayed step {t}")
        state, prev_bits = ref[:3], ref[3]
    h.close()


def test_delayed_update_skips_on_the_flag_and_guards_its_order(abi):
    n = 5000
    h = abi.Offload(2)
    dbuf = torch.empty(2 * n, dtype=torch.int16, device="cuda")
    staging = torch.empty(64 + 8 * 1024, dtype=torch.uint8, pin_memory=True)
    g, p, m, v = _inputs(n, "bf16", 3)
    hm, hmm, hv = (torch.from_numpy(a.copy()) for a in (p, m, v))
    dg = torch.from_numpy(g.view(np.int16).copy()).cuda()
    dparam = torch.full((n,), 9, dtype=torch.int16, device="cuda")
    dcoef = torch.ones(1, dtype=torch.float32, device="cuda")
    flag = torch.tensor([abi.ZERO_FLAG_NONFINITE_GRAD], dtype=torch.int32, device="cuda")
    with pytest.raises(abi.ZeroError) as e:                 # nothing has begun
        h.end(dparam)
    assert e.value.code == abi.ZERO_EINVAL
    h.begin(hm, hmm, hv, dg, "bf16", n, _abi_hp(abi, HP, 1), dcoef, flag, "bf16", dbuf, staging)
    with pytest.raises(abi.ZeroError) as e:                 # one update in flight at a time
        h.begin(hm, hmm, hv, dg, "bf16", n, _abi_hp(abi, HP, 1), dcoef, flag, "bf16", dbuf, staging)
    assert e.value.code == abi.ZERO_EINVAL
    assert h.end(dparam) is False                           # skipped: nothing moved
    assert np.array_equal(hm.numpy(), p) and np.all(dparam.cpu().numpy() == 9)
    h.close()


def test_delayed_end_refuses_its_own_buffer(abi):
    # The parameters in flight sit in the second half of the begin call's
    # device buffer; an end that would copy them onto that buffer is refused
    # and leaves the update in flight, and the next end applies it.
    n = 3000
    h = abi.Offload(2)
    dbuf = torch.empty(2 * n, dtype=torch.int16, device="cuda")
    staging = torch.empty(64 + 8 * 1024, dtype=torch.uint8, pin_memory=True)
    g, p, m, v = _inputs(n, "bf16", 5)
    hm, hmm, hv = (torch.from_numpy(a.copy()) for a in (p, m, v))
    dg = torch.from_numpy(g.view(np.int16).copy()).cuda()
    dcoef = torch.ones(1, dtype=torch.float32, device="cuda")
    dflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    h.begin(hm, hmm, hv, dg, "bf16", n, _abi_hp(abi, HP, 1), dcoef, dflag, "bf16", dbuf, staging)
    for bad in (dbuf[n:], dbuf[:n], dbuf[n // 2:n // 2 + n]):
        with pytest.raises(abi.ZeroError) as e:
            h.end(bad)
        assert e.value.code == abi.ZERO_EALIAS and h.in_flight
    dparam = torch.zeros(n, dtype=torch.int16, device="cuda")
    assert h.end(dparam) is True and not h.in_flight
    ref = step.adam_update(p, m, v, g, "bf16", HP, 1, np.float32(1.0), "bf16")
    adam_parity((hm.numpy(), hmm.numpy(), hv.numpy(), dparam.cpu().numpy().view(np.uint16)), ref, "bf16",
                "delayed step after a refused end")
    h.close()


def test_delayed_workload_lags_one_step_and_ends_equal(abi):
    # The shrunk 8-rank ZeRO-2 share with ZeRO-Offload, delayed and not: while
    # step t+1's reduce runs, the delayed run's device parameters are those of
    # step t-1; after its flush both runs hold the same state, bit for bit.
    import dataclasses
    from zero_sharded_mixed_flat_amd import runner, workloads
    shrink = dict(psi=8 * 200_001 + 5, units=(8 * 200_001 + 5,), max_norm=0.01)
    plain = runner.RankStep(dataclasses.replace(workloads.get("llama3_8b_nd8_z2_offload"), **shrink), seed=8)
    delayed = runner.RankStep(dataclasses.replace(workloads.get("llama3_8b_nd8_z2_offload_delayed"), **shrink), seed=8)
    history = [synth.bits(plain.param_out(0)).copy()]
    for t in range(1, 4):
        plain.step()
        delayed.step()
        torch.cuda.synchronize()
        history.append(synth.bits(plain.param_out(0)).copy())
        # the delayed run has ended step t-1's update only
        assert np.array_equal(synth.bits(delayed.param_out(0)), history[t - 1]), t
    assert delayed.flush() is True
    torch.cuda.synchronize()
    assert np.array_equal(synth.bits(delayed.param_out(0)), history[3])
    for a, b in ((plain.master, delayed.master), (plain.m, delayed.m), (plain.v, delayed.v)):
        assert np.array_equal(a.numpy().view(np.uint32), b.numpy().view(np.uint32))
    assert plain.counters()[:3] == delayed.counters()[:3] == (4, 3, 0)
