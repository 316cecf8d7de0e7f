"""A whole step captured as a HIP graph and replayed equals the eager step.

The captured AdamW reads its step-dependent scalars from device memory, which
each replay refreshes.  Every replay is compared bit for bit with an eager run
of the same workload and seed, with eager work and synchronisations between
the replays; the oracle parity of the eager step is covered elsewhere.
"""

import dataclasses

import numpy as np
import pytest
import torch

from zero_sharded_mixed_flat_amd import synth, workloads

pytestmark = pytest.mark.gpu

SHRUNK = {
    "tiny_nd4_z2": {},
    "llama3_8b_nd8_z2": dict(psi=8 * 200_001 + 5, units=(8 * 200_001 + 5,), max_norm=0.01),
    "paper_7p5b_nd64_z3_qwz8": dict(psi=6 * 156_250, units=(156_250,) * 6, max_norm=0.1),
    "gpt3_175b_nd16_z1": dict(psi=16 * 1_093_751, units=(16 * 1_093_751,), max_norm=0.05),
}


@pytest.fixture(scope="module")
def runner():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_sharded_mixed_flat_amd import runner as _runner
    return _runner


def _same(a, b, what):
    x = a.detach().view(torch.int32 if a.element_size() == 4 else torch.int16).cpu().numpy()
    y = b.detach().view(torch.int32 if b.element_size() == 4 else torch.int16).cpu().numpy()
    assert np.array_equal(x, y), what


@pytest.mark.parametrize("name", sorted(SHRUNK))
def test_graph_replays_equal_eager_steps(runner, name):
    w = dataclasses.replace(workloads.get(name), **SHRUNK[name])
    print(f"graph {name}", flush=True)
    eager = runner.RankStep(w, seed=21)
    graph = runner.RankStep(w, seed=21)
    graph.capture()
    torch.cuda.synchronize()
    for k in range(4):
        eager.step()
        graph.replay()
        # unrelated eager work between replays, then a synchronisation
        junk = torch.randn(1 << 20, device="cuda")
        assert torch.isfinite(junk.sum())
        torch.cuda.synchronize()
        for t in ("master", "m", "v"):
            _same(getattr(eager, t), getattr(graph, t), f"{t} after replay {k}")
        out_e = eager.full if eager.full is not None else eager.param
        out_g = graph.full if graph.full is not None else graph.param
        _same(out_e, out_g, f"16-bit parameters after replay {k}")
        if not w.pre_reduced:
            _same(eager.reduced, graph.reduced, f"reduced gradient after replay {k}")
        assert eager.norm.item() == graph.norm.item() and eager.coef.item() == graph.coef.item()
        assert int(graph.flag.item()) == 0
    assert graph.t == eager.t == 5
    if graph.codes is not None:
        _same(eager.codes, graph.codes, "codes")


def test_offload_cannot_be_captured(runner):
    w = dataclasses.replace(workloads.get("llama3_8b_nd8_z2_offload"), psi=8 * 1000, units=(8 * 1000,))
    with pytest.raises(ValueError):
        runner.RankStep(w, seed=1).capture()


def test_more_than_64_ranks_refuse_capture(runner):
    # Their pointer table is copied from host memory: captured, the copy would
    # keep a host address, so the call refuses before enqueueing anything.
    from zero_sharded_mixed_flat_amd import abi
    n, nd = 4096, 65
    contribs = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(nd)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(abi.zero_workspace_bytes(n, 1), dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(abi.ZeroError) as e:
        with torch.cuda.graph(g):
            abi.zero_reduce_shard(contribs, n, "bf16", 1.0, out, ws, 0, flag)
    assert e.value.code == abi.ZERO_EINVAL and "captured" in str(e.value)
    # eagerly, the same call works
    abi.zero_reduce_shard(contribs, n, "bf16", 1.0, out, ws, 0, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0 and not out.float().abs().sum().item()
