"""What one emulated rank holds, per role, against the pages' per-rank ledger.

`runner.allocation_plan` lists every buffer RankStep allocates with the role
it plays (RankStep checks its own allocations against that list on the GPU).
For the rank whose share runs, the 16-bit parameters, 16-bit gradients and
fp32 master/m/v must add up to the per-rank model state of its ZeRO stage --
4Ψ + 12Ψ/Nd (ZeRO-1), 2Ψ + 14Ψ/Nd (ZeRO-2), 16Ψ/Nd (ZeRO-3) (L3.2 显存优化与
ZeRO §2.3, the per-stage table; 026 notes §二) -- up to the partition's
padding and 4 KiB row alignment.  Buffers that stand in for the other ranks,
the ZeRO-3 gathered parameters and the workspace are outside the ledger.
The GPT-3-sized owner update materialises only the owner's working set: its
shard of gradients and parameters plus its fp32 state, 16Ψ/Nd.  Needs no GPU.
"""

import pytest

from oracle import accounting
from zero_sharded_mixed_flat_amd import abi, runner, workloads

OWN = ("params16", "grads16", "state32")


def _own_bytes(w):
    plan = abi.Plan(w.units, w.nd, w.stage, w.align)
    roles = runner.role_bytes(w, plan)
    n, _ = plan.rank(0)
    slack = 16 * (plan.full_numel() - w.psi) + 16 * (n * w.nd - w.psi) + 2 * runner.CONTRIB_ROW_ALIGN * 2
    return roles, sum(roles.get(r, 0) for r in OWN), slack


@pytest.mark.parametrize("name, stage", [("gpt2_1p5b_nd16_z1", 1), ("llama3_8b_nd8_z2", 2),
                                         ("paper_7p5b_nd64_z3", 3)])
def test_own_model_state_matches_the_stage_ledger(name, stage):
    w = workloads.get(name)
    assert w.stage == stage
    roles, own, slack = _own_bytes(w)
    expect = accounting.model_state_bytes(w.psi, w.nd, w.stage, 12)
    assert abs(own - expect) <= slack, (own, expect, slack)
    # per role as well: parameters, gradients, optimizer state
    p16 = {1: 2 * w.psi, 2: 2 * w.psi, 3: 2 * w.psi / w.nd}[stage]
    g16 = {1: 2 * w.psi, 2: 2 * w.psi / w.nd, 3: 2 * w.psi / w.nd}[stage]
    assert abs(roles["params16"] - p16) <= slack and abs(roles["grads16"] - g16) <= slack
    assert abs(roles["state32"] - 12 * w.psi / w.nd) <= slack


def test_workload_ledgers():
    # GPT-2 1.5B over 16 ranks under ZeRO-1: 4*1.5576e9 + 12*1.5576e9/16 = 7.398 GB;
    # 8.03e9 over 8 under ZeRO-2: 16.06 + 14.0525 = 30.1125 GB; the pages' 7.5B
    # over 64 ranks under ZeRO-3: 1.875 GB (printed as 1.88 GB, Lecture 18
    # notes §2.1 and 026 notes §四).
    for name, gb in (("gpt2_1p5b_nd16_z1", 7.398), ("llama3_8b_nd8_z2", 30.1125), ("paper_7p5b_nd64_z3", 1.875)):
        _, own, _ = _own_bytes(workloads.get(name))
        assert own / 1e9 == pytest.approx(gb, abs=0.001), name


def test_owner_update_subset():
    w = workloads.get("gpt3_175b_nd16_z1")
    roles, own, slack = _own_bytes(w)
    assert abs(own - 16 * w.psi / w.nd) <= slack                       # 175 GB
    assert own < accounting.model_state_bytes(w.psi, w.nd, 1, 12)      # a ZeRO-1 rank would hold 831.25 GB
    assert roles["grads16"] == roles["params16"] == 2 * (w.psi // w.nd)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_every_buffer_has_a_role(name):
    w = workloads.get(name)
    plan = abi.Plan(w.units, w.nd, w.stage, w.align)
    known = {"params16", "grads16", "state32", "state32_host", "peers", "gathered", "gather_codes", "work",
             "staging_host"}
    for buf, role, nbytes in runner.allocation_plan(w, plan):
        assert role.replace("all_ranks_", "") in known and nbytes > 0, (buf, role)
