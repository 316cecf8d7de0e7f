"""The seeded input generators: deterministic, chunk-independent, tiling exact."""

import numpy as np
import torch

from zero_sharded_mixed_flat_amd import synth


def test_same_seed_same_values():
    a = synth.grad16(10_000, "f16", 1e-3, seed=5, stream=3, device="cpu")
    b = synth.grad16(10_000, "f16", 1e-3, seed=5, stream=3, device="cpu")
    c = synth.grad16(10_000, "f16", 1e-3, seed=5, stream=4, device="cpu")
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_stream_seed_spreads():
    seeds = {synth.stream_seed(1, s, c) for s in range(50) for c in range(50)}
    assert len(seeds) == 2500 and all(0 <= s < 2 ** 63 for s in seeds)


def test_distributions_roughly_right():
    g = synth.grad16(1 << 18, "bf16", 1e-4, seed=1, stream=0, device="cpu").float()
    assert abs(float(g.std()) / 1e-4 - 1) < 0.02
    v = synth.state_f32(1 << 18, 1e-8, seed=1, stream=1, device="cpu", absolute=True)
    assert float(v.min()) >= 0
    o = synth.grad16(1 << 18, "f16", 1e-3, seed=1, stream=2, device="cpu",
                     outlier_frac=0.01, outlier_mult=100.0).float()
    frac_big = float((o.abs() > 0.01).float().mean())
    assert 0.005 < frac_big < 0.015


def test_tile():
    t = torch.arange(10, dtype=torch.float32)
    synth.tile_(t, 3)
    assert t.tolist() == [0, 1, 2, 0, 1, 2, 0, 1, 2, 0]


def test_bits_view():
    t = torch.tensor([1.0, -2.0], dtype=torch.float16)
    assert synth.bits(t).tolist() == [0x3C00, 0xC000]
    assert synth.bits(t).dtype == np.uint16
