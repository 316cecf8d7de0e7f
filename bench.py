"""Benchmark: one ZeRO rank's mixed-precision Adam step on one MI355X.

A step is the whole hot path over one batch of resident synthetic inputs:
reduce the rank's slice from its Nd contributions (with fused norm partials),
finalize the global norm and clip multiplier, run AdamW on the fp32 shard and
write the 16-bit parameters (plus the per-layer gather for ZeRO-3 workloads).

Prints ONE JSON line.  ``value`` is parameters updated per second by this GPU
(the whole job at one GPU).  ``roofline`` reports the dominant kernel (the
AdamW kernel: 28 algorithmic bytes per element) against MI355X's 8 TB/s HBM,
timed with HIP events on the stream the kernels run on.  ``cpu_baseline`` is
the CPU oracle timed on a bounded sample of the same workload's inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "zero_sharded_mixed_flat_amd", "csrc", "kernels.hip")


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counters.

    Only used when the counters were taken from the current kernel source.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def cpu_baseline(run, budget_s=12.0):
    """Time the CPU oracle on a bounded sample of this workload's own inputs."""
    import numpy as np

    from oracle import partition
    from oracle import step as ostep
    from oracle.step import AdamHparams
    from zero_sharded_mixed_flat_amd import synth

    w = run.w
    hp = AdamHparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.inv_loss_scale, w.max_norm)
    chunk = min(1 << 21, run.n)
    # Inputs: the first `chunk` elements of each contribution and of the state.
    if w.pre_reduced:
        grad = synth.bits(run.grad[:chunk])
        contribs = None
    else:
        contribs = [synth.bits(c[:chunk]) for c in run.contribs(0)]
    master = run.master[0, :chunk].cpu().numpy()
    m = run.m[0, :chunk].cpu().numpy()
    v = run.v[0, :chunk].cpu().numpy()
    elems, reps = 0, 0
    parity = None
    t0 = time.perf_counter()
    while True:
        if contribs is not None:
            reduced, _ = ostep.reduce_shard(contribs, w.grad_dtype)
        else:
            reduced = grad
        norm = ostep.norm_from_sumsq(ostep.sumsq_exact(reduced, w.grad_dtype, w.inv_loss_scale))
        coef = ostep.clip_coef(norm, w.max_norm)
        ostep.adam_update(master, m, v, reduced, w.grad_dtype, hp, 1, coef, w.param_dtype)
        if w.gather_per_unit:
            # the gather, on a one-unit sample layout whose slices are `chunk` long
            sample_plan = partition.make_plan([chunk * w.nd], w.nd, 3, 1)
            ostep.gather(sample_plan, [reduced] * w.nd, np.empty(chunk * w.nd, np.uint16))
        elems += chunk
        reps += 1
        if parity is None and contribs is not None:
            parity = bool(np.array_equal(reduced, synth.bits(run.reduced[0, :chunk])))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": elems / dt,
        "unit": "params/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{reps} x {chunk} owned elements of this workload's inputs (reduce over {w.nd} ranks, "
                  f"exact norm, AdamW{', gather' if w.gather_per_unit else ''}), single-threaded numpy",
        "seconds": round(dt, 3),
    }, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU exchange is design-only)", file=sys.stderr)
        return 2

    import torch

    from zero_sharded_mixed_flat_amd import runner, workloads

    name = args.workload or workloads.BENCH_DEFAULT
    w = workloads.get(name)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    _log(f"bench: allocating {name}")
    run = runner.RankStep(w, seed=args.seed)
    torch.cuda.synchronize()
    _log(f"bench: shard {run.n} elements, {args.warmup} warmup + {args.steps} timed steps")

    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()

    # Whole steps, wall clock bracketed by device synchronisation.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    # Per-kernel durations: HIP events on the stream the kernels are launched on.
    stream = torch.cuda.current_stream()
    phases = ["reduce", "norm", "adam", "gather"]
    acc = {p: 0.0 for p in phases}
    for _ in range(args.steps):
        ev = {p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for p in phases}
        run.flag.zero_()
        if not w.pre_reduced:
            ev["reduce"][0].record(stream)
            run.reduce_all()
            ev["reduce"][1].record(stream)
        ev["norm"][0].record(stream)
        run.norm_all()
        ev["norm"][1].record(stream)
        ev["adam"][0].record(stream)
        run.adam_all()
        ev["adam"][1].record(stream)
        if run.shards is not None:
            ev["gather"][0].record(stream)
            run.gather_all()
            ev["gather"][1].record(stream)
        run.t += 1
        torch.cuda.synchronize()
        for p in phases:
            if p == "reduce" and w.pre_reduced or p == "gather" and run.shards is None:
                continue
            acc[p] += ev[p][0].elapsed_time(ev[p][1])
    kern_ms = {p: acc[p] / args.steps for p in phases}

    owned = run.n * len(run.owners)
    alg_bytes = run.algorithmic_bytes()
    adam_bytes = 28 * owned
    adam_gbs = adam_bytes / (kern_ms["adam"] * 1e-3) / 1e9
    step_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    flag = int(run.flag.item())
    traffic = measured_traffic(name)

    result = {
        "metric": "sharded Adam step: params updated/s and achieved HBM GB/s (% of peak), 1 GPU",
        "value": owned / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": name, "psi": w.psi, "nd": w.nd, "zero_stage": w.stage, "rank": w.rank,
            "emulated_owners": len(run.owners), "shard_numel": run.n, "grad_dtype": w.grad_dtype,
            "param_dtype": w.param_dtype, "state_dtype": "f32", "parallelism": "one rank's share, 1 GPU",
        },
        "hbm_gbs": step_gbs,
        "hbm_frac_of_peak": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": alg_bytes,
        "kernel_ms": {k: round(v, 6) for k, v in kern_ms.items() if v > 0},
        "roofline": {
            "bound": "hbm",
            "kernel": "adam_kernel",
            "achieved": adam_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": adam_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": adam_bytes,
        },
        "step_flag": flag,
        "norm": float(run.norm.item()),
        "clip_coef": float(run.coef.item()),
    }
    if not args.no_cpu_baseline:
        _log("bench: timing the CPU oracle on a sample")
        cb, parity = cpu_baseline(run)
        result["cpu_baseline"] = cb
        result["sample_parity_reduced_bit_exact"] = parity
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
