"""The device AdamW gives the oracle's update, bit for bit, on edge inputs.

The oracle evaluates AdamW in fp64 from the fp32 inputs and rounds each
output once; so do the kernels, in the same order.  Both device entry points
(scalars passed as arguments, zero_adam_step; scalars read from device
memory, zero_adam_step_consts) are compared with `oracle.step.adam_update`,
at the parity bar (1e-9 + 1e-6 relative, one 16-bit ulp) and bit for bit, and
with the library's host AdamW on the same inputs: a step offloaded to the
host gives the same bits as one kept in HBM.  Inputs mix in zeros, fp32 and
16-bit subnormals and gradients whose square overflows fp32.
"""

import numpy as np
import pytest
import torch

from adam_inputs import edge_inputs
from oracle import step as ostep
from oracle.step import AdamHparams
from tolerance import adam_parity, adam_same

pytestmark = pytest.mark.gpu

TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}
HPS = {
    "adam": AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),
    "adamw": AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1),
    "scaled": AdamHparams(lr=6e-5, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.01, inv_loss_scale=2.0 ** -16),
}


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import abi as _abi
    return _abi


def _note(msg):
    print(msg, flush=True)


def _hp(abi, hp, t):
    return abi.adam_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.inv_loss_scale, t)


def _dev(a, offset, pad=8):
    """Device copy of a host array at element `offset` of a larger buffer."""
    host = torch.from_numpy(np.ascontiguousarray(a))
    buf = torch.zeros(a.size + offset + pad, dtype=host.dtype, device="cuda")
    buf[offset:offset + a.size].copy_(host)
    return buf[offset:offset + a.size]


class DeviceState:
    def __init__(self, p, m, v, pdt, offset, poffset):
        n = p.size
        self.n, self.pdt = n, pdt
        self.master, self.m, self.v = _dev(p, offset), _dev(m, offset), _dev(v, offset)
        pbuf = torch.zeros(n + poffset + 8, dtype=TORCH16[pdt], device="cuda")
        self.param = pbuf[poffset:poffset + n]
        self.offset = offset

    def step(self, abi, g_bits, gdt, hp, t, coef, via_consts):
        d_g = _dev(g_bits.view(np.int16), self.offset).view(TORCH16[gdt])
        d_coef = torch.tensor([coef], dtype=torch.float32, device="cuda")
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        h = _hp(abi, hp, t)
        if via_consts:
            c = abi.zero_adam_consts_fill(h)
            d_c = torch.tensor([getattr(c, name) for name, _ in abi.zero_adam_consts._fields_],
                               dtype=torch.float32, device="cuda")
            abi.zero_adam_step_consts(self.master, self.m, self.v, d_g, gdt, self.n, d_c, d_coef, flag,
                                      self.param, self.pdt)
        else:
            abi.zero_adam_step(self.master, self.m, self.v, d_g, gdt, self.n, h, d_coef, flag, self.param,
                               self.pdt)
        torch.cuda.synchronize()
        return (self.master.cpu().numpy(), self.m.cpu().numpy(), self.v.cpu().numpy(),
                self.param.view(torch.int16).cpu().numpy().view(np.uint16))


def _host_step(abi, g, p, m, v, gdt, pdt, hp, t, coef):
    n = g.size
    tp, tm, tv = (torch.from_numpy(a.copy()) for a in (p, m, v))
    tg = torch.from_numpy(g.view(np.int16).copy())
    out = torch.zeros(n, dtype=torch.int16)
    abi.zero_cpu_adam_step(tp, tm, tv, tg, gdt, n, _hp(abi, hp, t), coef, False, out, pdt, 4)
    return tp.numpy(), tm.numpy(), tv.numpy(), out.numpy().view(np.uint16)


def _oracle(p, m, v, g, gdt, hp, t, coef, pdt):
    with np.errstate(over="ignore"):          # v' of the largest bf16 gradients overflows fp32
        return ostep.adam_update(p, m, v, g, gdt, hp, t, coef, pdt)


@pytest.mark.parametrize("gdt, pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("hpname", sorted(HPS))
@pytest.mark.parametrize("n, offset, poffset", [
    (50_003, 0, 0),       # 16-byte vectors, ragged tail
    (50_003, 3, 3),       # peeled head, then vectors
    (20_001, 5, 2)])      # misalignments differ: every element on the scalar path
@pytest.mark.parametrize("via_consts", [False, True])
def test_device_adam_is_the_oracle_update(abi, gdt, pdt, hpname, n, offset, poffset, via_consts):
    hp = HPS[hpname]
    _note(f"adam bits {gdt}->{pdt} hp={hpname} n={n} off={offset}/{poffset} consts={via_consts}")
    g, p, m, v = edge_inputs(n, gdt, hp.inv_loss_scale, n + offset)
    t, coef = 4, np.float32(0.6180339)
    got = DeviceState(p, m, v, pdt, offset, poffset).step(abi, g, gdt, hp, t, coef, via_consts)
    adam_parity(got, _oracle(p, m, v, g, gdt, hp, t, coef, pdt), pdt, "vs oracle")
    adam_same(got, _host_step(abi, g, p, m, v, gdt, pdt, hp, t, coef), "vs host AdamW")


@pytest.mark.parametrize("gdt, pdt", [("bf16", "bf16"), ("f16", "f16")])
def test_five_steps_stay_bit_identical(abi, gdt, pdt):
    # Each side steps from its own previous state: identical sequences stay identical.
    hp = HPS["adamw"]
    n = 262_147
    _note(f"adam bits five steps {gdt}->{pdt} n={n}")
    g, p, m, v = edge_inputs(n, gdt, hp.inv_loss_scale, 5)
    dev = DeviceState(p, m, v, pdt, 0, 0)
    rng = np.random.default_rng(6)
    state = (p, m, v)
    for t in range(1, 6):
        if t > 1:
            g = rng.permutation(g)
        coef = np.float32(1.0 if t % 2 else 0.8125)
        got = dev.step(abi, g, gdt, hp, t, coef, via_consts=bool(t % 2))
        ref = _oracle(*state, g, gdt, hp, t, coef, pdt)
        adam_parity(got, ref, pdt, f"step {t}")
        state = ref[:3]
