"""Benchmark: one ZeRO rank's mixed-precision Adam step on one MI355X.

A step is the whole hot path over one batch of resident synthetic inputs:
reduce the rank's slice from its Nd contributions (with fused norm partials),
finalize the global norm and clip multiplier, run AdamW on the fp32 shard and
write the 16-bit parameters (plus the per-layer gather for ZeRO-3 workloads,
plain or block-quantised).

Prints ONE JSON line.  ``value`` is parameters updated per second by this GPU
(the whole job at one GPU).  ``roofline`` reports the dominant kernel (the
phase with the longest time per step: AdamW at 28 algorithmic bytes per
element on the default workload) against MI355X's 8 TB/s HBM, timed with HIP
events on the stream the kernels run on.  ``cpu_baseline`` is
the CPU oracle timed on a bounded sample of the same workload's inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--graph] [--flush-mb MB] [--no-cpu-baseline]
  --workload NAME   any workload of zero_sharded_mixed_flat_amd/workloads.py
  --graph           time replays of the step captured once as a HIP graph
  --flush-mb MB     touch MB MiB before each step (cold caches); time the steps alone
  --checkpoint DIR  instead: save and restore throughput of sharded optimizer state
  --summarize-trace / --summarize-counters  turn rocprofv3 output into profiles/ summaries
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
CSRC = os.path.join(ROOT, "zero_sharded_mixed_flat_amd", "csrc")
QUANT_KERNELS = ("quantize", "dequantize", "gather_dequant")
COPY_ELEMS = 1 << 31            # the reference copy: 4 GiB of 16-bit values
COPY_BYTES_EACH_WAY = 2 * COPY_ELEMS


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel):
    """Hash of the sources a kernel is built from (its file and the shared headers)."""
    own = "quant.hip" if kernel.startswith(QUANT_KERNELS) else "kernels.hip"
    h = hashlib.sha256()
    for name in (own, "device.h", "internal.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of one kernel of a workload from committed rocprofv3 counters.

    Only used while the kernel's sources hash as they did when the counters
    were taken.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload, {}).get("kernels", {}).get(kernel)
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    return entry.get("bytes_per_launch")


CPU_THREADS_MAX = 16


def cpu_baseline(run, budget_s=12.0):
    """Time the CPU oracle, as it stands, on a bounded sample of this workload's inputs.

    One thread per host core (at most 16), each running the oracle's step on
    its own chunk of the shard (chunks spread over the shard) until the time
    budget is spent; numpy releases the interpreter lock inside its array
    operations, so the threads run in parallel.
    """
    import threading

    import numpy as np

    from oracle import partition
    from oracle import quant as oquant
    from oracle import step as ostep
    from oracle.step import AdamHparams
    from zero_sharded_mixed_flat_amd import synth

    w = run.w
    hp = AdamHparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.inv_loss_scale, w.max_norm)
    threads = max(1, min(CPU_THREADS_MAX, len(os.sched_getaffinity(0))))
    chunk = min(1 << 20, run.n)
    offsets = [min(run.n - chunk, (k * run.n) // threads) // 8 * 8 for k in range(threads)]

    def inputs(o):
        if w.pre_reduced:
            contribs, grad = None, synth.bits(run.grad[o:o + chunk])
        else:
            contribs, grad = [synth.bits(c[o:o + chunk]) for c in run.contribs(0)], None
        state = tuple(t[0, o:o + chunk].cpu().numpy().copy() for t in (run.master, run.m, run.v))
        return contribs, grad, state

    samples = [inputs(o) for o in offsets]
    # The reduce writes in place over the rank's own contribution, so the
    # device's reduce of these very inputs is the next step's output.
    device_reduced = None
    if not w.pre_reduced:
        import torch
        run.step()
        torch.cuda.synchronize()
        device_reduced = synth.bits(run.reduced[0, offsets[0]:offsets[0] + chunk])
    counts = [0] * threads
    first_reduced = [None]
    stop = time.perf_counter() + budget_s

    def work(k):
        contribs, grad, (master, m, v) = samples[k]
        while True:
            reduced = grad if contribs is None else ostep.reduce_shard(contribs, w.grad_dtype)[0]
            norm = ostep.norm_from_sumsq(ostep.sumsq_exact(reduced, w.grad_dtype, w.inv_loss_scale))
            coef = ostep.clip_coef(norm, w.max_norm)
            _, _, _, param = ostep.adam_update(master, m, v, reduced, w.grad_dtype, hp, 1, coef, w.param_dtype)
            if w.gather_bits != 16:
                # quantise the owned chunk once, dequantise every rank's codes into the sample layout
                codes, scales = oquant.quantize(param, w.param_dtype, w.gather_bits)
                full = np.empty(chunk * w.nd, np.uint16)
                for r in range(w.nd):
                    full[r * chunk:(r + 1) * chunk] = oquant.dequantize(codes, scales, w.param_dtype)
            elif w.gather_per_unit:
                # the gather, on a one-unit sample layout whose slices are `chunk` long
                sample_plan = partition.make_plan([chunk * w.nd], w.nd, 3, 1)
                ostep.gather(sample_plan, [reduced] * w.nd, np.empty(chunk * w.nd, np.uint16))
            if k == 0 and first_reduced[0] is None:
                first_reduced[0] = reduced
            counts[k] += chunk
            if time.perf_counter() >= stop:
                return

    t0 = time.perf_counter()
    pool = [threading.Thread(target=work, args=(k,)) for k in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    dt = time.perf_counter() - t0
    parity = None
    if device_reduced is not None:
        parity = bool(np.array_equal(first_reduced[0], device_reduced))
    return {
        "value": sum(counts) / dt,
        "unit": "params/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{threads} threads, each on its own {chunk}-element chunk of this workload's inputs "
                  f"({sum(counts) // chunk} chunk steps: {_reduce_label(w)}, exact norm, "
                  f"AdamW{_gather_label(w)}), numpy",
        "seconds": round(dt, 3),
    }, parity


def host_copy_gbs(threads, nbytes=1 << 31):
    """Host memory copy bandwidth (read + write bytes per second / 1e9) with ``threads`` threads."""
    import torch
    saved = torch.get_num_threads()
    torch.set_num_threads(threads)
    try:
        a = torch.ones(nbytes // 4, dtype=torch.float32)
        b = torch.empty_like(a)
        b.copy_(a)
        best = float("inf")
        for _ in range(3):
            t0 = time.perf_counter()
            b.copy_(a)
            best = min(best, time.perf_counter() - t0)
        return 2 * nbytes / best / 1e9
    finally:
        torch.set_num_threads(saved)


def host_read_gbs(threads, nbytes=1 << 31):
    """Host memory read bandwidth (bytes per second / 1e9) with ``threads`` threads.

    A sum over a 2 GiB array: reads only, so no store pays the read-for-
    ownership a plain copy's destination does; the ceiling of a host kernel.
    """
    import torch
    saved = torch.get_num_threads()
    torch.set_num_threads(threads)
    try:
        a = torch.ones(nbytes // 4, dtype=torch.float32)
        a.sum()
        best = float("inf")
        for _ in range(3):
            t0 = time.perf_counter()
            a.sum()
            best = min(best, time.perf_counter() - t0)
        return nbytes / best / 1e9
    finally:
        torch.set_num_threads(saved)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _reduce_label(w):
    if w.pre_reduced:
        return "gradient arrives reduced (no reduce)"
    return f"reduce over {w.nd} ranks"


def _gather_label(w):
    if w.gather_bits != 16:
        return f", INT{w.gather_bits} quantise + {w.nd} dequantising gathers"
    return ", gather" if w.gather_per_unit else ""


def _rows(path):
    """The rows of a CSV file, read and closed."""
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name):
    name = name.replace("zf::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return name.replace("void ", "").split("(")[0]


def summarize_trace(stats_csv, command, bench_log=None):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run: its kernel
    statistics (this library's kernels first), then the same dispatches from
    the per-dispatch trace grouped by kernel and grid size, which separates
    launches of one kernel that do different work.  With ``bench_log`` (the
    output of the profiled bench.py run) it adds bench.py's own HIP-event
    time per launch of the roofline kernel in that same process beside
    rocprofv3's average for that kernel's busiest grid size."""
    from collections import defaultdict
    rows = _rows(stats_csv)
    ours = [r for r in rows if "zf::" in r["Name"]]
    other = [r for r in rows if "zf::" not in r["Name"]]
    out = ["# Kernel trace summary", "", "Command:", "", "```", command, "```", "",
           "rocprofv3 kernel statistics:", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in ours + other[:4]:
        out.append(f"| `{_short(r['Name'])[:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    if trace_csv != stats_csv and os.path.exists(trace_csv):
        groups = defaultdict(list)
        for r in _rows(trace_csv):
            if "zf::" in r["Kernel_Name"]:
                groups[(_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]))].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out += ["", "This library's dispatches by grid size (from the per-dispatch trace of the same run):", "",
                "| kernel | grid (threads) | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|---|"]
        for (name, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"| `{name}` | {grid} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
        if bench_log:
            out += _bench_agreement(bench_log, groups)
    return "\n".join(out) + "\n"


def _bench_agreement(bench_log, groups):
    """bench.py's JSON line from the profiled run against the trace of the same run."""
    with open(bench_log) as f:
        lines = [ln for ln in f if ln.startswith('{"metric"')]
    if not lines:
        raise RuntimeError(f"{bench_log} holds no bench.py result line")
    d = json.loads(lines[-1])
    rf = d["roofline"]
    out = ["", "bench.py's result line from the profiled run (the same process):", "",
           f"* `value` {d['value']:.4g} {d['unit']}, {d['ms_per_step']:.3f} ms per step "
           f"({d['steps']} steps after {d['warmup']} warmup)."]
    cands = [(k, v) for k, v in groups.items() if k[0].split("<")[0] == rf["kernel"]]
    if not cands:
        out.append(f"* roofline kernel `{rf['kernel']}` runs no GPU dispatch to compare.")
        return out
    (name, grid), durs = max(cands, key=lambda kv: sum(kv[1]))
    trace_us = sum(durs) / len(durs)
    hip_us = rf["launch_ms"] * 1e3
    out.append(f"* roofline kernel `{rf['kernel']}`: {hip_us:.1f} us per launch by HIP events on its stream "
               f"({rf['launches_per_step']} launch(es) per step; the events bracket the phase, so gaps between "
               f"launches count) against {trace_us:.1f} us average for `{name}` at grid {grid} in this trace: "
               f"ratio {hip_us / trace_us:.3f}. Achieved {rf['achieved']:.0f} {rf['unit']} of {rf['peak']:.0f} "
               f"(frac {rf['frac']:.3f}).")
    return out


def summarize_counters(fetch_csv, write_csv, phases, commands):
    """HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE, scaled by the reference copy.

    The reference copy is the 4 GiB -> 4 GiB gather dispatch in the same run;
    its known byte counts give one scale factor per counter.  ``phases`` is the
    workload's phase model (kernel, launches, algorithmic bytes per launch).
    Returns the markdown summary and the traffic entry of every phase kernel.
    """
    from collections import defaultdict
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        acc = defaultdict(list)
        for r in _rows(path):
            if r["Counter_Name"] != counter or "zf::" not in r["Kernel_Name"]:
                continue
            acc[(_short(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        per[counter] = {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}
    copy_grid = COPY_ELEMS // 8 // 2    # 16-byte pieces, two per lane: one lane per 16 elements
    copy_key = [k for k in per["FETCH_SIZE"] if k[0].startswith("gather_kernel") and k[1] == copy_grid]
    if not copy_key:
        raise RuntimeError("no reference copy dispatch in the counter files")
    ck = copy_key[0]
    ref_kib = COPY_BYTES_EACH_WAY / 1024
    fetch_scale = ref_kib / per["FETCH_SIZE"][ck][0]
    write_scale = ref_kib / per["WRITE_SIZE"][ck][0]
    out = ["# HBM byte counters", "", "Commands:", "", "```"] + list(commands) + ["```", "",
           f"Reference: the gather kernel copying {COPY_BYTES_EACH_WAY} bytes to another buffer "
           f"(grid {ck[1]}) read FETCH_SIZE {per['FETCH_SIZE'][ck][0]:.6g} KiB and WRITE_SIZE "
           f"{per['WRITE_SIZE'][ck][0]:.6g} KiB per dispatch, so the scale factors are "
           f"{fetch_scale:.5f} (fetch) and {write_scale:.5f} (write).", "",
           "| kernel | grid | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled bytes read "
           "| scaled bytes written | scaled total | algorithmic | ratio |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    by_prefix = {p["kernel"]: p for p in phases.values()}
    kernels = {}
    for k in sorted(per["FETCH_SIZE"], key=lambda k: -per["FETCH_SIZE"][k][0]):
        f, count = per["FETCH_SIZE"][k]
        w = per["WRITE_SIZE"].get(k, (float("nan"), 0))[0]
        rb, wb = f * 1024 * fetch_scale, w * 1024 * write_scale
        prefix = k[0].split("<")[0]
        phase = by_prefix.get(prefix) if k != ck else None
        alg = phase["bytes_per_launch"] if phase else None
        ratio = f"{(rb + wb) / alg:.4f}x" if alg else ""
        out.append(f"| `{k[0]}` | {k[1]} | {count} | {f:.6g} | {w:.6g} | {rb:.4g} | {wb:.4g} | {rb + wb:.4g} "
                   f"| {alg if alg is None else f'{alg:.4g}'} | {ratio} |")
        if phase and prefix not in kernels:
            kernels[prefix] = {"kernel": k[0], "grid": k[1], "bytes_per_launch": rb + wb, "bytes_read": rb,
                               "bytes_written": wb, "algorithmic_bytes_per_launch": alg,
                               "kernel_source_sha256_16": kernel_source_hash(prefix)}
    entry = {"fetch_scale": fetch_scale, "write_scale": write_scale, "kernels": kernels}
    return "\n".join(out) + "\n", entry


CKPT_WORKLOAD = "gpt2_1p5b_nd16_z1"


def checkpoint_bench(directory, name, seed):
    """Save every rank's fp32 state (one file per rank, flushed to disk), then
    restore the emulated rank's shard under the same partition and under half
    as many ranks.  Throughput counts the restored rank's bytes."""
    import shutil
    import tempfile

    import torch

    from zero_sharded_mixed_flat_amd import abi, runner, workloads

    w = workloads.get(name)
    run = runner.RankStep(w, seed=seed)
    run.step()
    torch.cuda.synchronize()
    n = run.n
    state = (run.master[0], run.m[0], run.v[0])
    per_rank = 3 * 4 * n
    staging = torch.empty(64 << 20, dtype=torch.uint8, pin_memory=True)
    work = tempfile.mkdtemp(prefix="zf-ckpt-", dir=directory)
    try:
        paths = [os.path.join(work, f"rank{r:04d}.zck") for r in range(w.nd)]
        _log(f"checkpoint: saving {w.nd} x {per_rank / 1e9:.2f} GB to {work}")
        save_s = []
        for r, path in enumerate(paths):   # the other ranks' files hold this rank's arrays, same sizes
            t0 = time.perf_counter()
            abi.zero_ckpt_save(path, run.plan, r, run.counters()[1], *state, staging)
            save_s.append(time.perf_counter() - t0)
        out = [torch.empty_like(state[0]) for _ in range(3)]
        t0 = time.perf_counter()
        abi.zero_ckpt_load(paths, run.plan, w.rank, *out, staging)
        same_s = time.perf_counter() - t0
        _, real = run.plan.rank(w.rank)
        exact = all(torch.equal(a[:real], b[:real]) for a, b in zip(out, state))
        half = abi.Plan(w.units, w.nd // 2, w.stage, w.align)
        n_half, _ = half.rank(0)
        out_half = [torch.empty(n_half, device="cuda") for _ in range(3)]
        t0 = time.perf_counter()
        abi.zero_ckpt_load(paths, half, w.rank // 2, *out_half, staging)
        half_s = time.perf_counter() - t0
        usage = shutil.disk_usage(work)
    finally:
        shutil.rmtree(work, ignore_errors=True)
    result = {
        "metric": "sharded checkpoint: save and restore of one rank's fp32 optimizer state",
        "unit": "GB/s",
        "workload": name,
        "bytes_per_rank": per_rank,
        "save_gbs_median": per_rank / sorted(save_s)[len(save_s) // 2] / 1e9,
        "save_gbs_min": per_rank / max(save_s) / 1e9,
        "restore_same_partition_gbs": per_rank / same_s / 1e9,
        "restore_resharded_gbs": 3 * 4 * n_half / half_s / 1e9,
        "reshard": f"{w.nd} -> {w.nd // 2} ranks, rank {w.rank // 2}",
        "restore_bit_exact": bool(exact),
        "durable": "fsync of each file and its directory before the save returns",
        "storage_free_gb": usage.free / 1e9,
        "data": "synthetic",
    }
    print(json.dumps(result), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-trace", metavar="STATS_CSV",
                    help="print a markdown summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--bench-line", metavar="LOG", default=None,
                    help="with --summarize-trace: the profiled bench.py run's output, to compare its timing")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarize FETCH_SIZE / WRITE_SIZE counter files, update profiles/traffic.json")
    ap.add_argument("--flush-mb", type=int, default=0,
                    help="touch a buffer of this many MiB before each timed step and time the steps alone with "
                         "HIP events (the step then starts with cold caches)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step as a HIP graph after the warmup and time its replays")
    ap.add_argument("--checkpoint", metavar="DIR",
                    help="time saving every rank's optimizer state to DIR and restoring one rank (same and "
                         "halved rank count); prints one JSON line")
    ap.add_argument("--command", action="append", default=[],
                    help="the command(s) that produced the files being summarized")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, "\n".join(args.command), args.bench_line), end="")
        return 0
    if args.summarize_counters:
        from zero_sharded_mixed_flat_amd import abi as _abi
        from zero_sharded_mixed_flat_amd import runner as _runner
        from zero_sharded_mixed_flat_amd import workloads as _wl
        name = args.workload or _wl.BENCH_DEFAULT
        w = _wl.get(name)
        phases = _runner.phase_model(w, _abi.Plan(w.units, w.nd, w.stage, w.align))
        text, entry = summarize_counters(*args.summarize_counters, phases, args.command)
        print(text, end="")
        if entry:
            try:
                with open(TRAFFIC_FILE) as f:
                    data = json.load(f)
            except (OSError, ValueError):
                data = {}
            data[name] = entry
            with open(TRAFFIC_FILE, "w") as f:
                json.dump(data, f, indent=1, sort_keys=True)
                f.write("\n")
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the step; --gpus {args.gpus} is not supported: "
              "the exchange between GPUs is not implemented", file=sys.stderr)
        return 2

    import torch

    from zero_sharded_mixed_flat_amd import runner, workloads

    name = args.workload or workloads.BENCH_DEFAULT
    w = workloads.get(name)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.checkpoint:
        return checkpoint_bench(args.checkpoint, args.workload or CKPT_WORKLOAD, args.seed)
    _log(f"bench: allocating {name}")
    run = runner.RankStep(w, seed=args.seed)
    torch.cuda.synchronize()
    _log(f"bench: shard {run.n} elements, {args.warmup} warmup + {args.steps} timed steps")

    for _ in range(args.warmup):
        run.step()
    run.flush()
    torch.cuda.synchronize()
    step_fn = run.step
    if args.graph:
        run.capture()
        run.replay()                     # one untimed replay
        torch.cuda.synchronize()
        step_fn = run.replay

    if args.flush_mb > 0:
        # Cold caches: a pass over the flush buffer before each step, which is
        # timed alone with HIP events; ms_per_step is their median.
        flush = torch.zeros(args.flush_mb << 20, dtype=torch.uint8, device="cuda")
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for a, b in pairs:
            flush.add_(1)
            a.record()
            step_fn()
            b.record()
        run.flush()
        torch.cuda.synchronize()
        cold = sorted(a.elapsed_time(b) for a, b in pairs)
        ms_per_step = cold[len(cold) // 2]
        del flush
    else:
        # Whole steps, wall clock bracketed by device synchronisation.
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step_fn()
        run.flush()                      # a delayed host update still in flight ends inside the timing
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = 1e3 * wall / args.steps

    # Per-kernel durations: HIP events on the stream the kernels are launched on.
    # Every step is enqueued before any is waited for, behind a few ms of
    # queued work, so the host runs ahead of the GPU and an event pair times
    # its kernels, not the host preparing the launch.  Where the host is the
    # slower side (a launch-bound workload) the gaps remain in the figures.
    stream = torch.cuda.current_stream()
    phases = ["reduce", "norm", "adam", "quantize", "gather"]
    acc = {p: 0.0 for p in phases}
    step_ms = []
    lead = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(10):
        lead.add_(1)
    events = []
    for _ in range(args.steps):
        ev = {p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for p in phases + ["step"]}
        events.append(ev)
        run._ensure_table()
        ev["step"][0].record(stream)
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
        if run.codes is not None:
            ev["quantize"][0].record(stream)
            run.quantize_all()
            ev["quantize"][1].record(stream)
        if run.shards is not None:
            ev["gather"][0].record(stream)
            run.gather_all()
            ev["gather"][1].record(stream)
        run.end_step()
        ev["step"][1].record(stream)
    torch.cuda.synchronize()
    del lead
    per_step = {p: [] for p in phases}
    for ev in events:
        step_ms.append(ev["step"][0].elapsed_time(ev["step"][1]))
        for p in phases:
            if (p == "reduce" and w.pre_reduced or p == "gather" and run.shards is None
                    or p == "quantize" and run.codes is None):
                continue
            per_step[p].append(ev[p][0].elapsed_time(ev[p][1]))
            acc[p] += per_step[p][-1]
    kern_ms = {p: acc[p] / args.steps for p in phases}

    # Plain-copy ceiling in the same run: the gather kernel on a one-unit,
    # one-owner plan is a pure copy of 4 GiB into another 4 GiB buffer, with
    # the same tiled non-temporal accesses as the step's kernels.  It is also
    # the reference of known size for scaling the HBM byte counters.
    from zero_sharded_mixed_flat_amd import abi
    copy_elems = COPY_ELEMS
    copy_plan = abi.Plan([copy_elems], 1, 3, 8)
    src = torch.empty(copy_elems, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    abi.zero_gather_params(copy_plan, [src], 0, 1, "f16", dst, run.ws)
    torch.cuda.synchronize()
    copy_ms = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        abi.zero_gather_params(copy_plan, [src], 0, 1, "f16", dst, run.ws)
        b.record(stream)
        torch.cuda.synchronize()
        copy_ms.append(a.elapsed_time(b))
    copy_bytes = 2 * 2 * copy_elems
    copy_gbs = copy_bytes / (sum(copy_ms) / len(copy_ms) * 1e-3) / 1e9
    del src, dst

    owned = run.n * len(run.owners)
    alg_bytes = run.algorithmic_bytes()
    step_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    t_next, applied, skipped, flag = run.counters()
    # The dominant kernel: the phase with the longest time per step.  Its
    # launches are timed together, so the per-launch time is the phase time
    # over its launch count (gaps between launches included).
    phase_model = run.phases()
    dom = max(phase_model, key=lambda p: kern_ms[p])
    dom_launch_ms = kern_ms[dom] / phase_model[dom]["launches"]
    dom_bytes = phase_model[dom]["bytes_per_launch"]
    dom_gbs = dom_bytes / (dom_launch_ms * 1e-3) / 1e9
    # Spread of the dominant kernel over the timed steps (GB/s per launch).
    dom_steps = sorted(dom_bytes / (t / phase_model[dom]["launches"] * 1e-3) / 1e9 for t in per_step[dom])
    dom_spread = {"min": dom_steps[0], "median": dom_steps[len(dom_steps) // 2], "max": dom_steps[-1],
                  "steps": len(dom_steps)}
    traffic = measured_traffic(name, phase_model[dom]["kernel"])
    roofline = {"bound": "hbm", "peak": HBM_PEAK_GBS, "peak_source": "MI355X published HBM3E bandwidth"}
    offload = None
    if phase_model[dom]["kernel"].startswith("host_"):
        # ZeRO-Offload: the dominant phase is the host AdamW, bound by host
        # memory; its ceiling is a host copy measured here with as many threads.
        # The ceiling is a host read: a plain copy pays a read of each destination
        # line before writing it, which the host AdamW's streamed output does not.
        host_gbs = host_copy_gbs(run.host_threads)
        read_gbs = host_read_gbs(run.host_threads)
        roofline = {"bound": "host_dram", "peak": read_gbs,
                    "peak_source": f"measured host read bandwidth, {run.host_threads} threads (no published figure)"}
        adam_ms = kern_ms["adam"]
        offload = {"delayed_update": bool(w.offload_delay),
                   "host_threads": run.host_threads, "host_isa": ["scalar", "avx2", "avx512"][abi.zero_cpu_isa()],
                   "host_adam_params_per_s": owned / (adam_ms * 1e-3),
                   "pcie_bytes_per_step": 4 * owned, "staging_bytes": run.staging.numel(),
                   "update_ms": adam_ms, "host_copy_gbs": host_gbs, "host_read_gbs": read_gbs, "cpu": cpu_model()}

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
        # arithmetic: the reduce adds in fp32, the norm and AdamW compute in fp64
        "dtype": "f64" if w.pre_reduced else "f32+f64",
        "data": "synthetic",
        "config": {
            "workload": name, "psi": w.psi, "nd": w.nd, "zero_stage": w.stage, "rank": w.rank,
            "emulated_owners": len(run.owners), "shard_numel": run.n, "grad_dtype": w.grad_dtype,
            "param_dtype": w.param_dtype, "state_dtype": "f32", "parallelism": "one rank's share, 1 GPU",
            "hip_graph": bool(args.graph),
            "caches": f"{args.flush_mb} MiB touched before each step" if args.flush_mb > 0 else "hot",
        },
        "hbm_gbs": step_gbs,
        "hbm_frac_of_peak": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": alg_bytes,
        "kernel_ms": {k: round(v, 6) for k, v in kern_ms.items() if v > 0},
        "step_ms_events": {"median": sorted(step_ms)[len(step_ms) // 2], "min": min(step_ms), "max": max(step_ms),
                           "steps": len(step_ms)},
        "copy_ceiling": {"kernel": "gather_kernel as a plain 4 GiB -> 4 GiB copy", "gbs": copy_gbs,
                         "frac_of_peak": copy_gbs / HBM_PEAK_GBS,
                         "step_frac_of_copy": step_gbs / copy_gbs,
                         "dominant_frac_of_copy": dom_gbs / copy_gbs},
        "roofline": {
            "bound": roofline["bound"],
            "kernel": phase_model[dom]["kernel"],
            "achieved": dom_gbs,
            "peak": roofline["peak"],
            "peak_source": roofline["peak_source"],
            "unit": "GB/s",
            "frac": dom_gbs / roofline["peak"],
            "achieved_per_step": dom_spread,
            "frac_per_step": {k: (v / roofline["peak"] if k != "steps" else v) for k, v in dom_spread.items()},
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
            "launch_ms": dom_launch_ms,
            "launches_per_step": phase_model[dom]["launches"],
        },
        "step_flag": flag,
        "steps_applied": applied,
        "steps_skipped": skipped,
        "norm": float(run.norm.item()),
        "clip_coef": float(run.coef.item()),
    }
    if offload:
        result["offload"] = offload
    if not args.no_cpu_baseline:
        _log("bench: timing the CPU oracle on a sample")
        cb, parity = cpu_baseline(run)
        cb["gbs"] = cb["value"] * alg_bytes / owned / 1e9   # the step's algorithmic bytes per parameter
        cb["cpu"] = cpu_model()
        result["cpu_baseline"] = cb
        result["sample_parity_reduced_bit_exact"] = parity
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
