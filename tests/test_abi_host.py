"""The C-ABI library on the host: it loads, exports every symbol the header
declares, its partitioner and accounting agree with the oracle exactly, and
invalid arguments are rejected before anything is launched (no GPU needed:
none of these calls reaches the HIP runtime)."""

import os
import random
import re

import pytest

from oracle import accounting, partition
from zero_sharded_mixed_flat_amd import abi, workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "zero_flat.h")


def _declared():
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z_]+)\s*\(", src)))


def test_header_declares_what_the_binding_knows():
    assert _declared() == sorted(abi.EXPORTED)


def test_library_exports_every_declared_symbol():
    for name in _declared():
        assert hasattr(abi.lib, name), name


def test_version():
    assert abi.zero_version() == 10301


@pytest.mark.parametrize("seed", range(60))
def test_partition_matches_oracle(seed):
    rng = random.Random(1000 + seed)
    units = [rng.choice([1, 7, 8, 9, rng.randint(1, 10 ** rng.randint(1, 9))])
             for _ in range(rng.randint(1, 8))]
    nd = rng.choice([1, 2, 3, 4, 5, 8, 16, 64, 100, 1024])
    stage = rng.choice([0, 1, 2, 3])
    align = rng.choice([1, 2, 8, 64])
    ours = abi.Plan(units, nd, stage, align)
    ref = partition.make_plan(units, nd, stage, align)
    info = ours.info()
    assert info["n_units"] == len(ref.units) and info["owners"] == ref.owners
    assert ours.full_numel() == ref.full_numel
    for i, u in enumerate(ref.units):
        assert ours.unit(i) == (u.numel, u.slice_numel, u.full_base, u.shard_base)
    for r in sorted({0, nd - 1, nd // 2, rng.randrange(nd)}):
        assert ours.rank(r) == (ref.shard_numel, ref.real_numel(r))
    # Tensor segments: split each unit into a few tensors.
    tensors = []
    for u in (units if stage == 3 else [sum(units)]):
        cuts = sorted(rng.sample(range(1, u), min(3, u - 1))) if u > 1 else []
        tensors += [b - a for a, b in zip([0] + cuts, cuts + [u])]
    for r in sorted({0, nd - 1, rng.randrange(nd)}):
        assert ours.segments(tensors, r) == partition.segments(ref, tensors, r)


def test_workload_layouts_match_oracle():
    for w in workloads.WORKLOADS.values():
        ours = abi.Plan(w.units, w.nd, w.stage, w.align)
        ref = partition.make_plan(w.units, w.nd, w.stage, w.align)
        assert ours.rank(w.rank) == (ref.shard_numel, ref.real_numel(w.rank)), w.name
        assert ours.full_numel() == ref.full_numel, w.name
        if w.tensors:
            assert ours.segments(w.tensors, w.rank) == partition.segments(ref, w.tensors, w.rank)


@pytest.mark.parametrize("stage", [0, 1, 2, 3])
@pytest.mark.parametrize("nd", [1, 4, 16, 64])
def test_accounting_matches_oracle(stage, nd):
    for psi in (1.0, 7.5e9, 175e9):
        for k in (12, 16):
            assert abi.zero_model_state_bytes(psi, nd, stage, k) == accounting.model_state_bytes(psi, nd, stage, k)
        assert abi.zero_comm_volume(psi, nd, stage) == pytest.approx(accounting.comm_volume(psi, nd, stage),
                                                                     rel=1e-15)


def test_plan_rejects_bad_arguments():
    for args in (([10], 0, 1, 8), ([10], 1025, 1, 8), ([10], 2, 4, 8), ([10], 2, 1, 0), ([0, 0], 2, 1, 8),
                 ([-1], 2, 1, 8)):
        with pytest.raises(abi.ZeroError) as e:
            abi.Plan(*args)
        assert e.value.code == abi.ZERO_EINVAL
    # the padded layout is bounded: 4096 one-element layers padded to 2^30 on
    # 1024 owners fill exactly 2^52 elements; one layer more is rejected
    assert abi.Plan([1] * 4096, 1024, 3, 1 << 30).full_numel() == 1 << 52
    with pytest.raises(abi.ZeroError) as e:
        abi.Plan([1] * 4097, 1024, 3, 1 << 30)
    assert e.value.code == abi.ZERO_EINVAL and "2^52" in str(e.value)
    assert abi.Plan([1 << 50], 1024, 1, 1 << 30).full_numel() == 1 << 50      # the largest real size
    p = abi.Plan([10, 20], 2, 3, 8)
    with pytest.raises(abi.ZeroError):
        p.segments([10, 21], 0)          # sizes do not add up
    with pytest.raises(abi.ZeroError):
        p.segments([15, 15], 0)          # a tensor crosses a unit
    with pytest.raises(abi.ZeroError):
        p.rank(2)


def test_workspace_bytes():
    # 8 KiB pointer table + 8 KiB of second-level sums + one fp64 partial sum
    # per 2048 elements and set (at least one per set).
    base = 16384
    assert abi.zero_workspace_bytes(0, 0) == base
    assert abi.zero_workspace_bytes(0, 1) == base + 8
    assert abi.zero_workspace_bytes(2048, 1) == base + 8
    assert abi.zero_workspace_bytes(2049, 3) == base + 3 * 2 * 8
    assert abi.zero_workspace_bytes(10 ** 10, 2) == base + 2 * (-(-10 ** 10 // 2048)) * 8
    with pytest.raises(abi.ZeroError):
        abi.zero_workspace_bytes(-1, 1)


# Fake, never-dereferenced device addresses: each call below must fail in
# validation, before the HIP runtime is touched.
A, B, W, F = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _reduce(**kw):
    args = dict(contribs=[A, A + 4096], n=1024, dtype=abi.ZERO_F16, inv_loss_scale=1.0, reduced_out=B,
                workspace=W, set_index=0, flag=F, stream=0,
                workspace_bytes=abi.zero_workspace_bytes(1024, 1))
    args.update(kw)
    return abi.zero_reduce_shard(**args)


@pytest.mark.parametrize("bad, code", [
    (dict(contribs=[]), abi.ZERO_EINVAL),
    (dict(n=-1), abi.ZERO_EINVAL),
    (dict(dtype=3), abi.ZERO_EINVAL),
    (dict(inv_loss_scale=0.3), abi.ZERO_EINVAL),
    (dict(inv_loss_scale=0.0), abi.ZERO_EINVAL),
    (dict(workspace_bytes=100), abi.ZERO_EINVAL),
    (dict(set_index=1), abi.ZERO_EINVAL),
    (dict(flag=0), abi.ZERO_EINVAL),
    (dict(reduced_out=B + 1), abi.ZERO_EINVAL),
    (dict(contribs=[A, 0]), abi.ZERO_EINVAL),
    (dict(reduced_out=A + 4096 + 2046), abi.ZERO_EALIAS),
    (dict(workspace=A + 64), abi.ZERO_EALIAS),
])
def test_reduce_rejects(bad, code):
    with pytest.raises(abi.ZeroError) as e:
        _reduce(**bad)
    assert e.value.code == code


def _adam(**kw):
    args = dict(master=A, m=A + 8192, v=A + 16384, grad=B, grad_dtype="bf16", n=1024,
                hp=abi.adam_hparams(3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, 1), coef=F, flag=F + 4,
                param_out=B + 8192, param_dtype="bf16", stream=0)
    args.update(kw)
    return abi.zero_adam_step(**args)


@pytest.mark.parametrize("bad, code", [
    (dict(n=-5), abi.ZERO_EINVAL),
    (dict(grad_dtype=0), abi.ZERO_EINVAL),
    (dict(hp=abi.adam_hparams(3e-4, 1.0, 0.95, 1e-8, 0.1, 1.0, 1)), abi.ZERO_EINVAL),
    (dict(hp=abi.adam_hparams(3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, 0)), abi.ZERO_EINVAL),
    (dict(hp=abi.adam_hparams(float("nan"), 0.9, 0.95, 1e-8, 0.1, 1.0, 1)), abi.ZERO_EINVAL),
    (dict(hp=abi.adam_hparams(3e-4, 0.9, 0.95, 1e-8, 0.1, 3.0, 1)), abi.ZERO_EINVAL),
    (dict(master=A + 2), abi.ZERO_EINVAL),
    (dict(coef=0), abi.ZERO_EINVAL),
    (dict(m=A + 4000), abi.ZERO_EALIAS),
    (dict(param_out=B + 100), abi.ZERO_EALIAS),
    (dict(param_out=A + 20000), abi.ZERO_EALIAS),
])
def test_adam_rejects(bad, code):
    with pytest.raises(abi.ZeroError) as e:
        _adam(**bad)
    assert e.value.code == code


def test_adam_zero_length_is_a_no_op():
    _adam(n=0, master=None, m=None, v=None, grad=None, param_out=None)


def _reduce_owners(**kw):
    args = dict(contribs=[A, A + 16384], n=1024, owners=3, contrib_stride=2048, dtype=abi.ZERO_F16,
                inv_loss_scale=1.0, reduced_out=B, reduced_stride=1024, workspace=W, flag=F, stream=0,
                workspace_bytes=abi.zero_workspace_bytes(1024, 3))
    args.update(kw)
    return abi.zero_reduce_owners(**args)


@pytest.mark.parametrize("bad, code", [
    (dict(owners=0), abi.ZERO_EINVAL),
    (dict(owners=1025), abi.ZERO_EINVAL),
    (dict(reduced_stride=1023), abi.ZERO_EINVAL),            # owners' outputs would overlap
    (dict(contrib_stride=-1), abi.ZERO_EINVAL),
    (dict(contrib_stride=(1 << 40) + 1), abi.ZERO_EINVAL),
    (dict(workspace_bytes=abi.zero_workspace_bytes(1024, 2)), abi.ZERO_EINVAL),   # room for 2 sets of 3
    (dict(reduced_out=A + 2 * 4096), abi.ZERO_EALIAS),        # inside rank 0's third owner's contribution
    (dict(workspace=B + 2 * 2048), abi.ZERO_EALIAS),           # inside the last owner's output
])
def test_reduce_owners_rejects(bad, code):
    with pytest.raises(abi.ZeroError) as e:
        _reduce_owners(**bad)
    assert e.value.code == code


def _adam_owners(**kw):
    n = 1024
    args = dict(master=A, m=A + 4 * 4 * n, v=A + 8 * 4 * n, state_stride=n, grad=B, grad_dtype="bf16",
                grad_stride=n, n=n, owners=4, table_dev=W, table_len=8, state_dev=W + 4096, coef=F, flag=F + 4,
                param_out=B + 2 * 4 * n, param_stride=n, param_dtype="bf16", stream=0)
    args.update(kw)
    return abi.zero_adam_step_owners(**args)


@pytest.mark.parametrize("bad, code", [
    (dict(owners=0), abi.ZERO_EINVAL),
    (dict(state_stride=1000), abi.ZERO_EINVAL),
    (dict(param_stride=1000), abi.ZERO_EINVAL),
    (dict(grad_stride=-4), abi.ZERO_EINVAL),
    (dict(table_len=0), abi.ZERO_EINVAL),
    (dict(table_dev=0), abi.ZERO_EINVAL),
    (dict(state_dev=W + 4100), abi.ZERO_EINVAL),              # not 8-byte aligned
    (dict(m=A + 3 * 4 * 1024), abi.ZERO_EALIAS),              # overlaps the last owner's master
    (dict(param_out=B + 2 * 3 * 1024), abi.ZERO_EALIAS),      # overlaps the last owner's gradient
    (dict(table_dev=A + 64), abi.ZERO_EALIAS),
    (dict(state_dev=A + 4 * 4096), abi.ZERO_EALIAS),
])
def test_adam_owners_rejects(bad, code):
    with pytest.raises(abi.ZeroError) as e:
        _adam_owners(**bad)
    assert e.value.code == code


def test_step_end_rejects():
    for flag, state, code in ((0, W, abi.ZERO_EINVAL), (F + 2, W, abi.ZERO_EINVAL), (F, W + 4, abi.ZERO_EINVAL),
                              (W + 16, W, abi.ZERO_EALIAS)):
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_step_end(flag, state, 0)
        assert e.value.code == code


def test_offload_handle_rejects_before_any_copy():
    h = abi.Offload(2)
    n = 1024
    args = dict(master=A, m=A + 4 * n, v=A + 8 * n, grad=B, grad_dtype="bf16", n=n,
                hp=abi.adam_hparams(3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, 1), coef=F, flag=F + 4, param_dtype="bf16",
                device_buffer=W, staging=0x50000000, stream=0, device_bytes=4 * n, staging_bytes=4096)
    for bad, code in ((dict(n=-1), abi.ZERO_EINVAL), (dict(device_bytes=4 * n - 2), abi.ZERO_EINVAL),
                      (dict(staging_bytes=100), abi.ZERO_EINVAL), (dict(staging=0x50000008), abi.ZERO_EINVAL),
                      (dict(device_buffer=B + 2 * n - 2), abi.ZERO_EALIAS), (dict(m=A + 4), abi.ZERO_EALIAS),
                      (dict(coef=0), abi.ZERO_EINVAL)):
        with pytest.raises(abi.ZeroError) as e:
            h.begin(**dict(args, **bad))
        assert e.value.code == code, bad
    with pytest.raises(abi.ZeroError) as e:              # nothing has begun
        h.end(B, stream=0)
    assert e.value.code == abi.ZERO_EINVAL
    h.close()
    with pytest.raises(abi.ZeroError):
        abi.Offload(0)


def test_grad_norm_rejects():
    base = dict(grad=None, n=100, dtype=1, inv_loss_scale=1.0, workspace=W, n_sets=1, extra_sumsq=None,
                n_extra=0, max_norm=1.0, flag=F, norm_out=F + 8, coef_out=F + 16, stream=0,
                workspace_bytes=abi.zero_workspace_bytes(100, 1))
    for bad in (dict(n_sets=0), dict(n_extra=2), dict(max_norm=float("inf")), dict(norm_out=F + 4),
                dict(workspace_bytes=8), dict(grad=B, dtype=7), dict(grad=W + 8)):
        args = dict(base, **bad)
        with pytest.raises(abi.ZeroError):
            abi.zero_grad_norm(**args)


def test_grad_norm_noalloc_rejects():
    # checked before any HIP call: a NULL gradient, n outside [0, 2^34]
    base = dict(grad=B, n=100, dtype=1, inv_loss_scale=1.0, extra_sumsq=None, n_extra=0, max_norm=1.0, flag=F,
                norm_out=F + 8, coef_out=F + 16, stream=0)
    for bad in (dict(grad=None), dict(n=abi.ZERO_NOALLOC_MAX_ELEMS + 1), dict(n=-1)):
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_grad_norm_noalloc(**dict(base, **bad))
        assert e.value.code == abi.ZERO_EINVAL, bad
    # its static scratch is exactly a one-set workspace at the largest n
    assert abi.ZERO_NOALLOC_SCRATCH_BYTES == abi.zero_workspace_bytes(abi.ZERO_NOALLOC_MAX_ELEMS, 1)


def test_gather_rejects():
    plan = abi.Plan([1000, 1000], 4, 3, 8)
    base = dict(plan=plan, shards=[A + i * 4096 for i in range(4)], unit_begin=0, unit_end=2, dtype=1,
                full=B, workspace=None, stream=0)
    for bad, code in ((dict(unit_end=3), abi.ZERO_EINVAL), (dict(unit_begin=2, unit_end=1), abi.ZERO_EINVAL),
                      (dict(dtype=9), abi.ZERO_EINVAL), (dict(full=A + 100), abi.ZERO_EALIAS),
                      (dict(shards=[A, 0, A, A]), abi.ZERO_EINVAL)):
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_gather_params(**dict(base, **bad))
        assert e.value.code == code
    abi.zero_gather_params(**dict(base, unit_begin=1, unit_end=1))   # empty range: no-op


def test_gather_rejects_above_64_owners():
    # The pointer table goes into the workspace: it must exist and overlap
    # neither the full buffer nor any shard.
    plan = abi.Plan([1000], 100, 3, 8)
    shard_bytes = 2 * plan.rank(0)[0]
    shards = [A + i * 4096 for i in range(100)]
    base = dict(plan=plan, shards=shards, unit_begin=0, unit_end=1, dtype=1, full=B, workspace=W, stream=0,
                workspace_bytes=abi.zero_workspace_bytes(0, 0))
    assert shard_bytes <= 4096
    for bad, code in ((dict(workspace=None, workspace_bytes=0), abi.ZERO_EINVAL),
                      (dict(workspace_bytes=100), abi.ZERO_EINVAL),
                      (dict(workspace=B + 64), abi.ZERO_EALIAS),
                      (dict(workspace=shards[57] + 16), abi.ZERO_EALIAS)):
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_gather_params(**dict(base, **bad))
        assert e.value.code == code, bad
    assert "workspace overlaps shard 57" in str(e.value)


def test_every_workload_fits_the_element_limit():
    for name, w in workloads.WORKLOADS.items():
        plan = abi.Plan(w.units, w.nd, w.stage, w.align)
        n, _ = plan.rank(0)
        assert n <= abi.ZERO_MAX_ELEMS, name
        assert all(plan.unit(u)[1] <= abi.ZERO_MAX_ELEMS for u in range(plan.info()["n_units"])), name


def test_sizes_beyond_the_element_limit_are_rejected():
    # No launch grid may exceed its hardware limit: every call refuses more
    # than ZERO_MAX_ELEMS elements before anything is enqueued.
    big = abi.ZERO_MAX_ELEMS + 1
    assert abi.zero_workspace_bytes(abi.ZERO_MAX_ELEMS, 1024) > 0
    with pytest.raises(abi.ZeroError):
        abi.zero_workspace_bytes(big, 1)
    ws = 1 << 45
    calls = [
        lambda: abi.zero_reduce_shard([A, A + 4096], big, abi.ZERO_F16, 1.0, B, W, 0, F, stream=0,
                                      workspace_bytes=ws),
        lambda: abi.zero_grad_norm(B, big, 1, 1.0, W, 1, None, 0, 1.0, F, F + 8, F + 16, stream=0,
                                   workspace_bytes=ws),
        lambda: _adam(n=big),
        lambda: abi.zero_quantize_blocks(A, "f16", big, 8, B, W, stream=0),
        lambda: abi.zero_dequantize_blocks(A, W, big, 8, B, "f16", stream=0),
        lambda: abi.zero_gather_params(abi.Plan([big], 1, 3, 8), [A], 0, 1, 1, B, None, stream=0),
        lambda: abi.zero_gather_dequant(abi.Plan([big + 255], 1, 3, 256), [A], [W], 0, 1, 8, 1, B, stream=0),
    ]
    for k, call in enumerate(calls):
        with pytest.raises(abi.ZeroError) as e:
            call()
        assert e.value.code == abi.ZERO_EINVAL and "2^34" in str(e.value), k


def test_quant_sizes():
    assert abi.zero_quant_code_bytes(1000, 8) == 1000
    assert abi.zero_quant_code_bytes(1001, 4) == 501
    assert abi.zero_quant_scale_count(0) == 0
    assert abi.zero_quant_scale_count(257) == 2
    with pytest.raises(abi.ZeroError):
        abi.zero_quant_code_bytes(10, 3)


def test_quant_rejects():
    for bad, code in ((dict(bits=3), abi.ZERO_EINVAL), (dict(dtype=5), abi.ZERO_EINVAL), (dict(x=A + 2), abi.ZERO_EINVAL),
                      (dict(codes=A + 1000), abi.ZERO_EALIAS), (dict(scales=A + 100), abi.ZERO_EALIAS)):
        args = dict(x=A, dtype=1, n=1000, bits=8, codes=B, scales=W, stream=0)
        args.update(bad)
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_quantize_blocks(**args)
        assert e.value.code == code
    with pytest.raises(abi.ZeroError):
        abi.zero_dequantize_blocks(B, W, 1000, 8, A + 4, 1, stream=0)      # y misaligned
    abi.zero_quantize_blocks(None, 1, 0, 8, None, None, stream=0)          # n = 0: no-op


def test_gather_dequant_rejects():
    plan = abi.Plan([4096, 2048], 4, 3, 8)                 # align 8: blocks could straddle
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_gather_dequant(plan, [A] * 4, [W] * 4, 0, 2, 8, 1, B, stream=0)
    assert e.value.code == abi.ZERO_EINVAL
    plan = abi.Plan([4096, 2048], 4, 3, 256)
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_gather_dequant(plan, [A] * 4, [W] * 4, 0, 2, 8, 1, B + 2, stream=0)   # full misaligned
    assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_gather_dequant(plan, [A] * 4, [W] * 4, 0, 2, 8, 1, B + 8, stream=0)   # full not 16-byte aligned
    assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_gather_dequant(plan, [A, A + 8, A, A], [W] * 4, 0, 2, 8, 1, B, stream=0)   # codes not 16-aligned
    assert e.value.code == abi.ZERO_EINVAL and "shard 1" in str(e.value)


def test_gather_dequant_rejects_above_64_owners():
    # Both pointer tables go into the workspace's first 16 KiB: it must exist
    # and overlap neither the full buffer nor any code or scale shard.
    plan = abi.Plan([256 * 100], 100, 3, 256)
    codes = [A + i * 4096 for i in range(100)]
    scales = [F + i * 64 for i in range(100)]
    base = dict(plan=plan, code_shards=codes, scale_shards=scales, unit_begin=0, unit_end=1, bits=8, dtype=1,
                full=B, workspace=W, stream=0, workspace_bytes=abi.zero_workspace_bytes(0, 0))
    for bad, code, text in ((dict(workspace=None, workspace_bytes=0), abi.ZERO_EINVAL, "workspace"),
                            (dict(workspace=B + 64), abi.ZERO_EALIAS, "full buffer"),
                            (dict(workspace=codes[70] - 1024), abi.ZERO_EALIAS, "overlaps shard 70"),
                            (dict(workspace=scales[99]), abi.ZERO_EALIAS, "overlaps shard 99")):
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_gather_dequant(**dict(base, **bad))
        assert e.value.code == code and text in str(e.value), (bad, str(e.value))


def test_pointer_table():
    import torch
    plan = abi.Plan([4096, 2048], 4, 3, 256)
    codes = abi.PointerTable([A, A + 16, A + 32, A + 48], 1 << 20)    # raw addresses are not size-checked
    scales = abi.PointerTable([W] * 4, 1 << 20)
    assert len(codes) == 4 and list(codes.array) == [A, A + 16, A + 32, A + 48]
    with pytest.raises(abi.ZeroError) as e:        # the table reaches the library's own checks
        abi.zero_gather_dequant(plan, codes, scales, 0, 2, 8, 1, B + 8, stream=0)
    assert "16-byte" in str(e.value)
    small = abi.PointerTable([torch.empty(0)] * 4, 0)
    with pytest.raises(ValueError):                # validated for fewer bytes than the call needs
        abi.zero_gather_params(plan, small, 0, 2, "f16", None, stream=0)
    with pytest.raises(ValueError):                # host tensors are refused when the table is built
        abi.PointerTable([torch.empty(8)], 32, "shard")
