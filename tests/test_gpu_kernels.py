"""GPU parity: every kernel through the C ABI against the oracle.

Sizes span several blocks and ragged tails; views at odd element offsets take
the peeled-head path, views with mismatched offsets the scalar path.  Inputs
come from seeded generators on the host; expected values come only from
``oracle``.  Bars: reduced 16-bit gradients bit-exact; the norm within 1e-5
relative and the derived fp64 bound (about 5e-15), the clip coefficient
within one fp32 ulp; master/m/v within 1e-9 + 1e-6 relative, 16-bit params
within one ulp, and both bit for bit (see ``tolerance``).
"""

import numpy as np
import pytest
import torch

from oracle import partition, rounding, step
from oracle.step import AdamHparams
from tolerance import adam_parity, coef_ok, norm_ok

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


def _rand16(rng, n, std, dtype):
    return rounding.narrow((rng.standard_normal(n) * std).astype(np.float32), dtype)


def _dev16(bits, dtype, pad=0, offset=0):
    """Device copy of uint16 patterns, placed at element `offset` of a buffer."""
    buf = torch.zeros(len(bits) + offset + pad, dtype=TORCH16[dtype], device="cuda")
    host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH16[dtype])
    buf[offset:offset + len(bits)].copy_(host)
    return buf[offset:offset + len(bits)]


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _ws(abi, n, sets):
    return torch.empty(abi.zero_workspace_bytes(n, sets), dtype=torch.uint8, device="cuda")


def _scalars():
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    coef = torch.zeros(1, dtype=torch.float32, device="cuda")
    return flag, norm, coef


# ---------------------------------------------------------------------------
# a1 reduce (+ a2 finalize on its partials)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nd", [1, 2, 3, 4, 5, 8, 16, 32, 64, 100])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 4099, 300_001])
def test_reduce_and_norm(abi, dtype, nd, n):
    _note(f"reduce dtype={dtype} nd={nd} n={n}")
    rng = np.random.default_rng(nd * 1_000_003 + n + (0 if dtype == "f16" else 7))
    std = 1e-3 if dtype == "f16" else 1e-4
    contribs = [_rand16(rng, n, std, dtype) for _ in range(nd)]
    ref, bad = step.reduce_shard(contribs, dtype) if n else (np.zeros(0, np.uint16), False)
    dev = [_dev16(c, dtype) for c in contribs]
    out = torch.empty(n, dtype=TORCH16[dtype], device="cuda")
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    abi.zero_reduce_shard(dev, n, dtype, 1.0, out, ws, 0, flag)
    abi.zero_grad_norm(None, n, dtype, 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), ref)
    assert int(flag.item()) == 0 and not bad
    ref_norm = step.norm_from_sumsq(step.sumsq_exact(ref, dtype)) if n else 0.0
    got = float(norm.item())
    norm_ok(got, ref_norm, n)
    coef_ok(coef.item(), step.clip_coef(ref_norm, 1.0))


@pytest.mark.parametrize("nd", [1000, 1024])
@pytest.mark.parametrize("n", [4099, 300_001])
def test_reduce_maximum_rank_count(abi, nd, n):
    # Up to ZERO_MAX_RANKS contributions: the pointer table lives in the
    # workspace and the mean divides (1000) or multiplies by 2^-10 (1024).
    dtype = "bf16"
    _note(f"reduce nd={nd} n={n}")
    rng = np.random.default_rng(nd + n)
    contribs = [_rand16(rng, n, 1e-4, dtype) for _ in range(nd)]
    ref, bad = step.reduce_shard(contribs, dtype)
    dev = [_dev16(c, dtype) for c in contribs]
    out = torch.empty(n, dtype=TORCH16[dtype], device="cuda")
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    abi.zero_reduce_shard(dev, n, dtype, 1.0, out, ws, 0, flag)
    abi.zero_grad_norm(None, n, dtype, 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), ref) and not bad
    norm_ok(norm.item(), step.norm_from_sumsq(step.sumsq_exact(ref, dtype)), n)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("offsets", [(1, 1, 1), (3, 3, 3), (1, 2, 1), (0, 0, 5)])
def test_reduce_misaligned(abi, dtype, offsets):
    # (1,1,1) / (3,3,3): common misalignment -> peeled head + vector body;
    # mismatched offsets -> scalar path.  Same answer either way.
    n, nd = 70_013, 4
    _note(f"reduce misaligned dtype={dtype} offsets={offsets}")
    rng = np.random.default_rng(17)
    contribs = [_rand16(rng, n, 1e-3, dtype) for _ in range(nd)]
    ref, _ = step.reduce_shard(contribs, dtype)
    dev = [_dev16(c, dtype, offset=offsets[0] if i % 2 == 0 else offsets[1]) for i, c in enumerate(contribs)]
    outbuf = torch.empty(n + 8, dtype=TORCH16[dtype], device="cuda")
    out = outbuf[offsets[2]:offsets[2] + n]
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    abi.zero_reduce_shard(dev, n, dtype, 1.0, out, ws, 0, flag)
    abi.zero_grad_norm(None, n, dtype, 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), ref)
    norm_ok(norm.item(), step.norm_from_sumsq(step.sumsq_exact(ref, dtype)), n)


def test_reduce_subnormals_and_loss_scale(abi):
    # fp16 values around the subnormal range, scaled by 65536 and unscaled in
    # the norm by 2**-16; every output bit must match.
    n, nd = 100_000, 16
    _note("reduce subnormals + loss scale")
    rng = np.random.default_rng(23)
    contribs = [_rand16(rng, n, 1e-6, "f16") for _ in range(nd // 2)]
    contribs += [_rand16(rng, n, 1e-3 * 65536, "f16") for _ in range(nd // 2)]
    ref, _ = step.reduce_shard(contribs, "f16")
    dev = [_dev16(c, "f16") for c in contribs]
    out = torch.empty(n, dtype=torch.float16, device="cuda")
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    abi.zero_reduce_shard(dev, n, "f16", 2.0 ** -16, out, ws, 0, flag)
    abi.zero_grad_norm(None, n, "f16", 2.0 ** -16, ws, 1, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), ref)
    norm_ok(norm.item(), step.norm_from_sumsq(step.sumsq_exact(ref, "f16", 2.0 ** -16)), n)


def test_reduce_rank_order_case(abi):
    # The hand-worked rank-order case: 65504, 3*2**-24, -65504 averages to 0.
    _note("reduce rank-order case")
    vals = [np.array([65504.0] * 9, np.float32), np.array([3 * 2.0 ** -24] * 9, np.float32),
            np.array([-65504.0] * 9, np.float32)]
    contribs = [rounding.narrow(v, "f16") for v in vals]
    dev = [_dev16(c, "f16") for c in contribs]
    out = torch.empty(9, dtype=torch.float16, device="cuda")
    ws = _ws(abi, 9, 1)
    flag, _, _ = _scalars()
    abi.zero_reduce_shard(dev, 9, "f16", 1.0, out, ws, 0, flag)
    torch.cuda.synchronize()
    assert np.all(_bits(out) == 0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("where", [0, 8, 12_345, 99_999])
def test_reduce_flags_nonfinite(abi, dtype, where):
    n, nd = 100_000, 8
    _note(f"reduce nonfinite dtype={dtype} where={where}")
    rng = np.random.default_rng(29)
    contribs = [_rand16(rng, n, 1e-3, dtype) for _ in range(nd)]
    contribs[3][where] = 0x7C00 if dtype == "f16" else 0x7F80       # +inf
    contribs[5][(where * 7) % n] = 0xFE00 if dtype == "f16" else 0xFFC0   # NaN
    ref, bad = step.reduce_shard(contribs, dtype)
    assert bad
    dev = [_dev16(c, dtype) for c in contribs]
    out = torch.empty(n, dtype=TORCH16[dtype], device="cuda")
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    abi.zero_reduce_shard(dev, n, dtype, 1.0, out, ws, 0, flag)
    abi.zero_grad_norm(None, n, dtype, 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    f = int(flag.item())
    assert f & abi.ZERO_FLAG_NONFINITE_GRAD and f & abi.ZERO_FLAG_NONFINITE_NORM
    got = _bits(out)
    fin = rounding.is_finite16(ref, dtype)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(rounding.is_finite16(got, dtype), fin)


def test_reduce_is_deterministic(abi):
    n, nd = 1_000_003, 8
    _note("reduce determinism")
    rng = np.random.default_rng(31)
    dev = [_dev16(_rand16(rng, n, 1e-4, "bf16"), "bf16") for _ in range(nd)]
    norms = []
    for _ in range(3):
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        ws = _ws(abi, n, 1)
        flag, norm, coef = _scalars()
        abi.zero_reduce_shard(dev, n, "bf16", 1.0, out, ws, 0, flag)
        abi.zero_grad_norm(None, n, "bf16", 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
        torch.cuda.synchronize()
        norms.append((norm.item(), ws.cpu().numpy().tobytes()[16384:]))   # partial sums
    assert norms[0] == norms[1] == norms[2]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nd, k, n, offset", [(4, 0, 300_001, 0), (8, 7, 4099, 0), (3, 1, 100_003, 3),
                                               (64, 30, 20_000, 1), (100, 99, 5_001, 0)])
def test_reduce_in_place_over_one_contribution(abi, dtype, nd, k, n, offset):
    # reduced_out may be contribution k itself: each element is read from every
    # rank before it is written, so the result is the oracle's, and the other
    # contributions are untouched.
    _note(f"reduce in place dtype={dtype} nd={nd} k={k} n={n} offset={offset}")
    rng = np.random.default_rng(nd * 31 + k + n)
    contribs = [_rand16(rng, n, 1e-3, dtype) for _ in range(nd)]
    ref, bad = step.reduce_shard(contribs, dtype)
    dev = [_dev16(c, dtype, offset=offset) for c in contribs]
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    abi.zero_reduce_shard(dev, n, dtype, 1.0, dev[k], ws, 0, flag)
    abi.zero_grad_norm(None, n, dtype, 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert not bad and int(flag.item()) == 0
    assert np.array_equal(_bits(dev[k]), ref)
    for r in range(nd):
        if r != k:
            assert np.array_equal(_bits(dev[r]), contribs[r]), r
    norm_ok(norm.item(), step.norm_from_sumsq(step.sumsq_exact(ref, dtype)), n)


@pytest.mark.parametrize("n, sets", [(20_000_003, 1), (5_000_001, 4)])
def test_norm_two_stage_finalize(abi, n, sets):
    # More than 8192 partial sums: the finalize folds them in two stages.
    _note(f"two-stage norm n={n} sets={sets}")
    rng = np.random.default_rng(n + sets)
    grads = [_rand16(rng, n, 1e-3, "bf16") for _ in range(sets)]
    ws = _ws(abi, n, sets)
    flag, norm, coef = _scalars()
    outs = []
    for i, g in enumerate(grads):
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        abi.zero_reduce_shard([_dev16(g, "bf16")], n, "bf16", 1.0, out, ws, i, flag)
        outs.append(out)
    abi.zero_grad_norm(None, n, "bf16", 1.0, ws, sets, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    first = norm.item()
    abi.zero_grad_norm(None, n, "bf16", 1.0, ws, sets, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert norm.item() == first                                   # same tree every time
    ref = step.norm_from_sumsq(sum(step.sumsq_exact(g, "bf16") for g in grads))
    norm_ok(first, ref, n * sets)
    for g, out in zip(grads, outs):
        assert np.array_equal(_bits(out), g)                      # nd = 1 is the identity


@pytest.mark.parametrize("n, offset", [(20_000_003, 0), (17_000_001, 3), (16_777_216 + 2048 * 3, 1)])
def test_prereduced_norm_large(abi, n, offset):
    # The partials pass over one array at sizes with more than 8192 partial
    # sums (two-stage finalize), aligned and misaligned.
    _note(f"prereduced norm n={n} offset={offset}")
    rng = np.random.default_rng(n)
    g = _rand16(rng, n, 1e-4, "bf16")
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    dg = _dev16(g, "bf16", offset=offset)
    abi.zero_grad_norm(dg, n, "bf16", 1.0, ws, 1, None, 0, 0.5, flag, norm, coef)
    torch.cuda.synchronize()
    ref = step.norm_from_sumsq(step.sumsq_exact(g, "bf16"))
    norm_ok(norm.item(), ref, n)
    coef_ok(coef.item(), step.clip_coef(ref, 0.5))
    assert int(flag.item()) == 0


# ---------------------------------------------------------------------------
# a2 standalone partials pass + extra partial sums
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n", [1, 1000, 777_777])
def test_grad_norm_prereduced(abi, dtype, n):
    _note(f"grad_norm prereduced dtype={dtype} n={n}")
    rng = np.random.default_rng(n)
    g = _rand16(rng, n, 1e-2, dtype)
    extra = np.array([0.25, 3.5], np.float64)
    dg = _dev16(g, dtype, offset=n % 3)
    ws = _ws(abi, n, 1)
    flag, norm, coef = _scalars()
    dev_extra = torch.from_numpy(extra).cuda()
    abi.zero_grad_norm(dg, n, dtype, 1.0, ws, 1, dev_extra, 2, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    ref = step.norm_from_sumsq(step.sumsq_exact(g, dtype) + 0.25 + 3.5)
    norm_ok(norm.item(), ref, n, n_extra=2)
    coef_ok(coef.item(), step.clip_coef(ref, 1.0))
    assert int(flag.item()) == 0


def test_grad_norm_clipping_disabled_and_empty(abi):
    ws = _ws(abi, 0, 1)
    flag, norm, coef = _scalars()
    g = torch.empty(0, dtype=torch.float16, device="cuda")
    abi.zero_grad_norm(g, 0, "f16", 1.0, ws, 1, None, 0, 1.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert norm.item() == 0.0 and coef.item() == 1.0
    g = _dev16(_rand16(np.random.default_rng(1), 5000, 1.0, "f16"), "f16")
    ws = _ws(abi, 5000, 1)
    abi.zero_grad_norm(g, 5000, "f16", 1.0, ws, 1, None, 0, 0.0, flag, norm, coef)
    torch.cuda.synchronize()
    assert norm.item() > 1.0 and coef.item() == 1.0


# ---------------------------------------------------------------------------
# a3 Adam
# ---------------------------------------------------------------------------

HPS = {
    "c1": AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1),
    "c0": AdamHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),
    "c3": AdamHparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, inv_loss_scale=2.0 ** -16),
}


def _hp(abi, hp, t):
    return abi.adam_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.inv_loss_scale, t)


@pytest.mark.parametrize("gdt, pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("hpname", ["c1", "c0", "c3"])
@pytest.mark.parametrize("n, offset, poffset", [
    (1, 0, 0), (9, 0, 0), (262_147, 0, 0),
    (100_003, 3, 3),      # common misalignment: peeled head, then 16-byte vectors
    (50_001, 5, 2)])      # param offset differs: scalar path
def test_adam(abi, gdt, pdt, hpname, n, offset, poffset):
    hp = HPS[hpname]
    _note(f"adam {gdt}->{pdt} hp={hpname} n={n} off={offset}/{poffset}")
    rng = np.random.default_rng(n + offset)
    scale = 1.0 / hp.inv_loss_scale
    g = _rand16(rng, n, 1e-3 * scale, gdt)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    coef = np.float32(0.6180339)
    t = 3
    p_ref, m_ref, v_ref, bits_ref = step.adam_update(master, m, v, g, gdt, hp, t, coef, pdt)

    def dev32(a):
        buf = torch.zeros(n + offset + 4, dtype=torch.float32, device="cuda")
        buf[offset:offset + n].copy_(torch.from_numpy(a))
        return buf[offset:offset + n]

    d_master, d_m, d_v = dev32(master), dev32(m), dev32(v)
    d_g = _dev16(g, gdt, offset=offset)
    pbuf = torch.zeros(n + poffset + 8, dtype=TORCH16[pdt], device="cuda")
    d_p = pbuf[poffset:poffset + n]
    d_coef = torch.tensor([coef], dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    abi.zero_adam_step(d_master, d_m, d_v, d_g, gdt, n, _hp(abi, hp, t), d_coef, flag, d_p, pdt)
    torch.cuda.synchronize()
    got = (d_master.cpu().numpy(), d_m.cpu().numpy(), d_v.cpu().numpy(), _bits(d_p))
    adam_parity(got, (p_ref, m_ref, v_ref, bits_ref), pdt, "adam")


def test_adam_skips_when_flagged(abi):
    n = 10_000
    _note("adam skip")
    rng = np.random.default_rng(2)
    master = torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).cuda()
    m = torch.from_numpy((rng.standard_normal(n) * 1e-5).astype(np.float32)).cuda()
    v = torch.from_numpy(np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)).cuda()
    g = _dev16(_rand16(rng, n, 1e-3, "f16"), "f16")
    p = torch.full((n,), 7.0, dtype=torch.float16, device="cuda")
    before = [x.clone() for x in (master, m, v, p)]
    coef = torch.ones(1, dtype=torch.float32, device="cuda")
    for bit in (abi.ZERO_FLAG_NONFINITE_GRAD, abi.ZERO_FLAG_NONFINITE_NORM):
        flag = torch.tensor([bit], dtype=torch.int32, device="cuda")
        abi.zero_adam_step(master, m, v, g, "f16", n, _hp(abi, HPS["c0"], 1), coef, flag, p, "f16")
        torch.cuda.synchronize()
        for a, b in zip((master, m, v, p), before):
            assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# a4 gather
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("units, nd, align", [
    ([1000, 37, 2050], 4, 8), ([4096] * 5, 8, 8), ([999, 1], 100, 8), ([1001, 33], 3, 1), ([64] * 3, 64, 8)])
def test_gather(abi, units, nd, align):
    _note(f"gather units={units} nd={nd} align={align}")
    plan = abi.Plan(units, nd, 3, align)
    ref_plan = partition.make_plan(units, nd, 3, align)
    rng = np.random.default_rng(len(units) * 1000 + nd)
    shards = [rng.integers(0, 1 << 16, ref_plan.shard_numel, dtype=np.uint32).astype(np.uint16)
              for _ in range(nd)]
    dev = [_dev16(s, "f16") for s in shards]
    full = torch.full((ref_plan.full_numel,), 0.5, dtype=torch.float16, device="cuda")
    ws = _ws(abi, 0, 0)
    # One unit first, then the remaining units in one call.
    abi.zero_gather_params(plan, dev, 1, 2, "f16", full, ws)
    torch.cuda.synchronize()
    expect = np.full(ref_plan.full_numel, 0x3800, np.uint16)      # 0.5 in fp16
    step.gather(ref_plan, shards, expect, 1, 2)
    assert np.array_equal(_bits(full), expect)
    abi.zero_gather_params(plan, dev, 0, len(units), "f16", full, ws)
    torch.cuda.synchronize()
    step.gather(ref_plan, shards, expect)
    assert np.array_equal(_bits(full), expect)


@pytest.mark.parametrize("quantised", [False, True])
def test_pointer_tables_may_be_reused_at_once(abi, quantised):
    # With more than 64 owners the shard pointers reach the kernel through a
    # table copied into the workspace.  The call reads the caller's arrays
    # before it returns: a caller that points its (pinned) arrays at other
    # valid shards at once, while the stream is still busy, still gets the
    # gather of the shards it passed.
    import ctypes
    _note(f"pointer tables reused at once, quantised={quantised}")
    units, nd, align = [2560, 768], 100, 256
    plan = abi.Plan(units, nd, 3, align)
    ref_plan = partition.make_plan(units, nd, 3, align)
    n = ref_plan.shard_numel
    rng = np.random.default_rng(7)
    sets = [[rounding.narrow((rng.standard_normal(n) * 0.02).astype(np.float32), "bf16") for _ in range(nd)]
            for _ in range(2)]
    dev = [[_dev16(x, "bf16") for x in shards] for shards in sets]
    if quantised:
        cb, nb = abi.zero_quant_code_bytes(n, 8), abi.zero_quant_scale_count(n)
        codes = [[torch.empty(cb, dtype=torch.uint8, device="cuda") for _ in range(nd)] for _ in range(2)]
        scales = [[torch.empty(nb, dtype=torch.float32, device="cuda") for _ in range(nd)] for _ in range(2)]
        for k in range(2):
            for r in range(nd):
                abi.zero_quantize_blocks(dev[k][r], "bf16", n, 8, codes[k][r], scales[k][r])
        arrays = [[[t.data_ptr() for t in codes[k]], [t.data_ptr() for t in scales[k]]] for k in range(2)]
    else:
        arrays = [[[t.data_ptr() for t in dev[k]]] for k in range(2)]
    tables = [torch.tensor(a, dtype=torch.int64).pin_memory() for a in arrays[0]]   # the caller's arrays, pinned
    full = torch.zeros(ref_plan.full_numel, dtype=torch.bfloat16, device="cuda")
    ws = _ws(abi, 0, 0)
    torch.cuda.synchronize()
    busy = torch.zeros(1 << 28, dtype=torch.uint8, device="cuda")
    for _ in range(8):                        # queued work: the stream is busy when the call returns
        busy.add_(1)
    stream = torch.cuda.current_stream().cuda_stream
    as_ptrs = [ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_void_p)) for t in tables]
    if quantised:
        rc = abi.lib.zero_gather_dequant(plan.handle, as_ptrs[0], as_ptrs[1], 0, 2, 8, abi.ZERO_BF16,
                                         full.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    else:
        rc = abi.lib.zero_gather_params(plan.handle, as_ptrs[0], 0, 2, abi.ZERO_BF16, full.data_ptr(),
                                        ws.data_ptr(), ws.numel(), stream)
    for t, a in zip(tables, arrays[1]):
        t.copy_(torch.tensor(a, dtype=torch.int64))       # at once: now the other, equally valid, shards
    torch.cuda.synchronize()
    assert rc == abi.ZERO_OK, abi.zero_last_error()
    assert busy[0].item() == 8
    got = _bits(full)
    if quantised:
        from oracle import quant
        coded = [quant.quantize(x, "bf16", 8) for x in sets[0]]
        shards = [quant.dequantize(c, sc, "bf16") for c, sc in coded]
    else:
        shards = sets[0]
    expect = np.zeros(ref_plan.full_numel, np.uint16)
    step.gather(ref_plan, shards, expect)
    assert np.array_equal(got, expect)
