#!/usr/bin/env python3
"""Benchmark of one rank's sharded AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over the rank's slice: the host layout call
(shard_layout: flatten, floor-rule slice, segment table) and the fused GPU step
(adamw_shard_step: rank-order fp32 reduction of the F bf16 contributions, AdamW on the fp32
master / m / v, bf16 copy into the flat parameter layout).  Inputs are synthetic, seeded and
resident in HBM before the timed region; the gradient buffers are drawn once and re-read by every
step.  The timed region is K steps bracketed by device synchronisation; each kernel launch is also
bracketed by HIP events on the stream it runs on, which gives the kernel's own average duration
for the roofline figure.

Prints one JSON line (the last line of stdout).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "params updated/sec per GPU (sharded AdamW step); achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
DEFAULT_WORKLOAD = "dense7b_n8_rank0"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "fsdp_sharded_optimizer_layout_amd", "csrc", "shard_step.hip")
RESHARD_SOURCE = os.path.join(ROOT, "fsdp_sharded_optimizer_layout_amd", "csrc", "reshard.hip")
STEP_KERNEL = "void (anonymous namespace)::fused_step_kernel"
RESHARD_KERNEL = "(anonymous namespace)::reshard_kernel"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes_per_param(fan_in):
    """HBM bytes one real parameter must move in the fused step: F bf16 contributions read,
    fp32 master / m / v each read and written, one bf16 parameter written."""
    return 2 * fan_in + 3 * 4 * 2 + 2


def algorithmic_bytes_per_param_f32grad():
    """The fused step fed by an fp32 gradient shard: 4 B gradient read, 24 B state, 2 B bf16."""
    return 4 + 3 * 4 * 2 + 2


def source_digest(source=KERNEL_SOURCE):
    """Digest of a kernel source with comments and whitespace removed: the counter figures stay
    valid across comment edits and lapse with any change to the code."""
    import re
    with open(source) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def counter_traffic(key, source=KERNEL_SOURCE):
    """Per-launch HBM bytes from the committed rocprofv3 counter summary, if it was taken on the
    kernel source as it is now (otherwise None)."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(key)
    if not entry or entry.get("kernel_source_sha256_16") != source_digest(source):
        return None
    return entry.get("bytes_per_launch")


def reshard_key(workload, dst_world, dst_pad, dst_rank):
    return f"reshard:{workload}:{dst_world}:{dst_pad}:{dst_rank}"


def summarize_counters(key, fetch_dir, write_dir, kernel_prefix=STEP_KERNEL, source=KERNEL_SOURCE,
                       calib_kernel="stream_copy_kernel", calib_bytes=4 << 30):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch) into per-launch HBM bytes of the measured kernel, each counter scaled by what it
    reads for the plain copy kernel, whose true traffic is calib_bytes read and calib_bytes
    written.  Writes the result into profiles/traffic.json under `key`."""
    import csv
    import statistics

    def per_dispatch(d, counter):
        path = os.path.join(d, "run_counter_collection.csv")
        step, calib = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                kib = float(r["Counter_Value"])
                if r["Kernel_Name"].startswith(kernel_prefix):
                    step.append(kib)
                elif calib_kernel in r["Kernel_Name"]:
                    calib.append(kib)
        return statistics.median(step), statistics.median(calib), len(step)

    f_step, f_cal, nf = per_dispatch(fetch_dir, "FETCH_SIZE")
    w_step, w_cal, nw = per_dispatch(write_dir, "WRITE_SIZE")
    f_scale = calib_bytes / (f_cal * 1024.0)
    w_scale = calib_bytes / (w_cal * 1024.0)
    fetch = f_step * 1024.0 * f_scale
    write = w_step * 1024.0 * w_scale
    try:
        with open(PROFILE_TRAFFIC) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    rec[key] = {
        "bytes_per_launch": round(fetch + write),
        "fetch_bytes": round(fetch), "write_bytes": round(write),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "dispatches": [nf, nw],
        "kernel_source_sha256_16": source_digest(source),
    }
    with open(PROFILE_TRAFFIC, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec[key]))


def cpu_baseline(workload, seconds=12.0, sample=1 << 21):
    """The oracle as it is, single-threaded NumPy on the host, on the first `sample` elements of
    the same workload's slice; repeated steps until about `seconds` of work."""
    import numpy as np
    import workloads as W
    from oracle import layout as OL
    from oracle import step as OS

    w = W.WORKLOADS[workload]
    lo, hi, osegs = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    n = min(sample, hi - lo)
    flags = np.zeros(n, dtype=np.int64)
    for s in osegs:
        a, b = s["shard_begin"], min(n, s["shard_begin"] + s["length"])
        if a < n:
            flags[a:b] = s["flags"]
    master, m, v = W.np_state(w, n, 0)
    grads = W.np_grads(w, n, 1, 0)
    steps = 0
    t0 = time.perf_counter()
    while True:
        steps += 1
        master, m, v, out = OS.shard_step(master, m, v, grads, flags, w.hp, steps)
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    n_real = int(np.count_nonzero((flags & OL.PADDING) == 0))
    return {"value": n_real * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} elements of the {workload} slice, fan-in {w.fan_in}, "
                      f"{steps} oracle steps in {el:.1f} s (NumPy float32, one thread)"}


def _oracle_chunk(args):
    """Worker of the parallel baseline: the oracle on elements [a, b) of the sampled slice."""
    workload, a, b, seconds = args
    import numpy as np
    import workloads as W
    from oracle import layout as OL
    from oracle import step as OS

    w = W.WORKLOADS[workload]
    lo, hi, osegs = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    flags = np.zeros(b - a, dtype=np.int64)
    for s in osegs:
        x, y = max(a, s["shard_begin"]), min(b, s["shard_begin"] + s["length"])
        if x < y:
            flags[x - a:y - a] = s["flags"]
    master, m, v = W.np_state(w, b - a, a)
    grads = W.np_grads(w, b - a, 1, a)
    steps = 0
    t0 = time.perf_counter()
    while True:
        steps += 1
        master, m, v, _ = OS.shard_step(master, m, v, grads, flags, w.hp, steps)
        if time.perf_counter() - t0 >= seconds:
            break
    return int(np.count_nonzero((flags & OL.PADDING) == 0)) * steps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_parallel(workload, procs, seconds=12.0, chunk=1 << 20):
    """The same oracle in `procs` processes, each stepping its own contiguous chunk of the slice
    (valid because the step is elementwise once the layout is fixed).  Rate = all processes'
    real parameters x steps / the wall time of the whole pool."""
    import multiprocessing as mp

    import workloads as W
    from oracle import layout as OL

    w = W.WORKLOADS[workload]
    lo, hi, _ = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    n = hi - lo
    procs = max(1, min(procs, n // chunk if n >= chunk else 1))
    jobs = [(workload, i * chunk, min(n, (i + 1) * chunk), seconds) for i in range(procs)]
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(procs) as pool:
        done = sum(pool.map(_oracle_chunk, jobs))
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "params/s", "cores": procs, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{procs} processes, each stepping the oracle on its own "
                      f"{chunk}-element chunk of the {workload} slice for about {seconds:.0f} s "
                      f"(NumPy float32); rate over the pool's wall time including start-up"}


def copy_reference(F, torch, dev, stream, nbytes=4 << 30):
    """Plain 16-byte copy of nbytes (non-temporal loads and stores): the bandwidth a pure
    read+write stream reaches, and the calibration kernel of the counter runs."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        F.stream_copy(src, dst, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    reps = 10
    for _ in range(reps):
        F.stream_copy(src, dst, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    copy_ms = a.elapsed_time(b) / reps
    ref = {"GBps": round(2 * nbytes / (copy_ms / 1e3) / 1e9, 1), "bytes_moved": 2 * nbytes,
           "kernel": "fsdpshard_stream_copy (16-byte loads and stores)"}
    log(f"copy reference: {ref['GBps']} GB/s")
    del src, dst
    return ref


def cpu_baseline_reshard(workload, dst_pad, dst_world, seconds=12.0):
    """The oracle's reshard as it is (NumPy, one thread) on one decoder layer of the workload's
    tensors: all destination shards of that layer from the source shards, repeated for about
    `seconds`.  Rate in destination elements per second."""
    import numpy as np
    import workloads as W
    from oracle import layout as OL
    from oracle import reshard as OR

    w = W.WORKLOADS[workload]
    sizes = w.sizes[1:10] if len(w.sizes) > 10 else w.sizes
    offs, P = OL.flatten_offsets(sizes, w.pad_multiple)
    flat = np.zeros(P, dtype=np.float32)
    rng = np.random.default_rng(0)
    for o, n in zip(offs, sizes):
        flat[o:o + n] = rng.standard_normal(n, dtype=np.float32)
    src = OR.shard(flat, sizes, w.pad_multiple, w.world_size)
    del flat
    reps, produced = 0, 0
    t0 = time.perf_counter()
    while True:
        out = OR.reshard(src, sizes, w.pad_multiple, dst_pad, dst_world)
        produced += sum(o.size for o in out)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": produced / el, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sizes)} tensors ({P} flat elements, fp32) of {workload}, "
                      f"{w.world_size} -> {dst_world} ranks, padding {w.pad_multiple} -> "
                      f"{dst_pad}, all destination shards, {reps} repetitions in {el:.1f} s"}


def bench_reshard(args, w, F, W, torch):
    """Reshard path: one destination rank's fp32 optimizer state (master, m, v) built from the
    source ranks' shards.  A step is the host plan plus three reshard_copy launches; the source
    shards it reads are resident in HBM (only the ranks the plan touches are allocated)."""
    dst_pad = args.reshard_pad or w.pad_multiple
    dst_world, dst_rank = args.reshard_world, args.reshard_rank
    pieces = F.reshard_plan(w.sizes, w.pad_multiple, w.world_size, dst_pad, dst_world, dst_rank)
    Ld, _ = F.shard_layout(w.sizes, dst_world, dst_rank, dst_pad)
    n_dst = Ld.n
    src_elems = [F.shard_layout(w.sizes, w.world_size, r, w.pad_multiple)[0].n
                 for r in range(w.world_size)]
    used = sorted({int(r) for r in pieces["src_rank"] if r >= 0})
    real = int(pieces["length"][pieces["src_rank"] >= 0].sum())
    log(f"reshard {w.name}: {w.world_size} ranks pad {w.pad_multiple} -> {dst_world} ranks pad "
        f"{dst_pad}, rank {dst_rank}: {n_dst} elements, {len(pieces)} pieces, source ranks {used}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    states = []
    for j in range(3):
        g = torch.Generator(device=dev)
        g.manual_seed(100 + j)
        src = [torch.randn(src_elems[r], dtype=torch.float32, device=dev, generator=g)
               if r in used else None for r in range(w.world_size)]
        dst = torch.empty(n_dst, dtype=torch.float32, device=dev)
        states.append((src, dst))
    torch.cuda.synchronize()
    bytes_per_launch = 4 * (real + n_dst)   # real elements read and all destination elements written

    def one_step(ev=None):
        p = F.reshard_plan(w.sizes, w.pad_multiple, w.world_size, dst_pad, dst_world, dst_rank)
        for j, (src, dst) in enumerate(states):
            if ev is not None:
                ev[j][0].record(stream)
            F.reshard_copy(src, dst, p, stream=stream)
            if ev is not None:
                ev[j][1].record(stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in states] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(events[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    ms = [events[i][j][0].elapsed_time(events[i][j][1])
          for i in range(args.steps) for j in range(len(states))]
    avg = sum(ms) / len(ms)
    achieved = bytes_per_launch / (avg / 1e3) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; reshard_copy avg {avg:.3f} ms, "
        f"{achieved:.1f} GB/s")
    copy_ref = None
    if not args.no_copy_reference:
        del states
        torch.cuda.empty_cache()
        copy_ref = copy_reference(F, torch, dev, stream)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline_reshard(w.name, dst_pad, dst_world)
        log(f"cpu oracle: {cpu['value']:.3e} elements/s")
    rec = {
        "metric": "optimizer-state elements resharded/sec per GPU; achieved HBM GB/s vs peak",
        "value": round(3 * n_dst / (ms_per_step / 1e3), 1),
        "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {
            "workload": w.name, "path": "reshard",
            "src": {"world_size": w.world_size, "pad_multiple": w.pad_multiple},
            "dst": {"world_size": dst_world, "pad_multiple": dst_pad, "rank": dst_rank,
                    "elems": n_dst},
            "pieces": len(pieces), "source_ranks": used, "real_elems": real,
            "states": "fp32 master, m, v (three reshard_copy launches per step)",
            "kernel_avg_ms": round(avg, 4), "kernel_min_ms": round(min(ms), 4),
            "algorithmic_bytes_per_launch": bytes_per_launch,
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": counter_traffic(reshard_key(w.name, dst_world, dst_pad, dst_rank),
                                                RESHARD_SOURCE)},
        "copy_reference": copy_ref,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--groups-per-wave", type=int, default=0,
                    help="512-element groups per wavefront (1, 2, 4; 0 = library default)")
    ap.add_argument("--path", choices=["fused", "clipped", "clipped32", "accumulate", "split",
                                       "reshard"],
                    default="fused",
                    help="fused: the fused step (default); clipped: sum of squares + clipped "
                         "step; clipped32: reduction fused with the sum of squares into an fp32 "
                         "shard + clipped fp32-gradient step; accumulate: fp32 micro-batch "
                         "accumulation (the last fused with the sum of squares) + clipped fp32 "
                         "step; "
                         "split: the step without its bf16 output, then unflatten_bf16; "
                         "reshard: move one destination rank's fp32 master/m/v to another "
                         "world size and padding multiple")
    ap.add_argument("--reshard-world", type=int, default=6,
                    help="reshard path: destination world size")
    ap.add_argument("--reshard-pad", type=int, default=0,
                    help="reshard path: destination padding multiple (0 = the workload's)")
    ap.add_argument("--reshard-rank", type=int, default=1,
                    help="reshard path: destination rank")
    ap.add_argument("--micro-batches", type=int, default=4)
    ap.add_argument("--state", choices=["blocked", "separate"], default="blocked",
                    help="optimizer-state layout: one array of 512-element blocks of master, m "
                         "and v (default), or three separate arrays (the split path always uses "
                         "separate arrays)")
    ap.add_argument("--max-grad-norm", type=float, default=1.0)
    ap.add_argument("--evict-mb", type=int, default=-1,
                    help="MiB written between timed steps to flush the 256 MB last-level cache "
                         "(-1: 1024 when one step moves under 2 GB, else 0); with eviction the "
                         "per-step time is the sum of the step's HIP-event kernel times")
    ap.add_argument("--cpu-procs", type=int, default=16,
                    help="processes for the parallel oracle baseline (0: skip it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-reference", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        if args.path == "reshard":
            import workloads as W
            w = W.WORKLOADS[args.workload]
            key = reshard_key(w.name, args.reshard_world, args.reshard_pad or w.pad_multiple,
                              args.reshard_rank)
            summarize_counters(key, *args.summarize_counters, kernel_prefix=RESHARD_KERNEL,
                               source=RESHARD_SOURCE)
        else:
            summarize_counters(args.workload, *args.summarize_counters)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: it times one rank's slice on a single MI355X and "
              "has no multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fsdp_sharded_optimizer_layout_amd as F
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    F.lib()  # fail loudly if the library is missing
    if args.groups_per_wave:
        F.set_groups_per_wave(args.groups_per_wave)

    w = W.WORKLOADS[args.workload]
    if args.path == "reshard":
        bench_reshard(args, w, F, W, torch)
        return
    L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    n, lo, Fi = L.n, L.lo, w.fan_in
    log(f"workload {w.name}: P={L.P} slice [{L.lo}, {L.hi}) n={n} n_real={L.n_real} "
        f"F={Fi} segments={L.n_segments}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    master, m, v = W.torch_state(w, n, 0, dev)
    grads = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(Fi)]
    W.torch_grads_into(w, grads, 1, 0)
    if w.nan_padding_grads:
        for s in segs:
            if s["flags"] & F.SEG_PADDING:
                for g in grads:
                    g[int(s["shard_begin"]): int(s["shard_begin"] + s["length"])] = 0x7FC0
    phase = lo % 8
    flat = torch.empty(n + phase, dtype=torch.int16, device=dev)
    segs_dev = F.segments_to_device(segs, dev)
    blocked = args.state == "blocked" and args.path != "split"
    if blocked:
        state = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device=dev)
        F.state_to_blocked(master, m, v, state)
        torch.cuda.synchronize()
        del master, m, v

        def step_bf16(t, **kw):
            F.adamw_shard_step_blocked(state, grads, step=t, n=n, **kw)

        def step_f32(acc, t, **kw):
            F.adamw_shard_step_f32grad_blocked(state, acc, step=t, n=n, **kw)
    else:
        def step_bf16(t, **kw):
            F.adamw_shard_step(master, m, v, grads, step=t, **kw)

        def step_f32(acc, t, **kw):
            F.adamw_shard_step_f32grad(master, m, v, acc, step=t, **kw)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    bpp = algorithmic_bytes_per_param(Fi)
    common = dict(segs=segs_dev, n_segments=L.n_segments, flat=flat, flat_index0=lo - phase,
                  lo=lo, stream=stream, **w.hp)

    # Stages of one step: (name, launch(t), algorithmic bytes per launch).  The fused path is the
    # default; the clipped and accumulate paths measure the clipping and micro-batch rows.
    stages = []
    if args.path == "fused":
        stages.append(("adamw_shard_step" + ("_blocked" if blocked else ""),
                       lambda t: step_bf16(t, **common), L.n_real * bpp))
    elif args.path == "split":
        no_out = {k: v for k, v in common.items() if k not in ("flat", "flat_index0", "lo")}
        stages.append(("adamw_shard_step (no bf16 output)", lambda t: F.adamw_shard_step(
            master, m, v, grads, step=t, **no_out), L.n_real * (bpp - 2)))
        stages.append(("unflatten_bf16", lambda t: F.unflatten_bf16(
            master, flat, flat_index0=lo - phase, lo=lo, segs=segs_dev,
            n_segments=L.n_segments, stream=stream), L.n_real * 4 + n * 2))
    else:
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        ws = torch.empty(max(8, F.grad_sumsq_workspace_bytes(n)), dtype=torch.uint8, device=dev)
        if args.path == "clipped":
            stages.append(("grad_sumsq_shard", lambda t: F.grad_sumsq_shard(
                sumsq, contribs=grads, n=n, segs=segs_dev, n_segments=L.n_segments,
                workspace=ws, stream=stream), n * 2 * Fi))
            stages.append(("adamw_shard_step (clipped)", lambda t: step_bf16(
                t, max_grad_norm=args.max_grad_norm, grad_sumsq=sumsq, **common), L.n_real * bpp))
        elif args.path == "clipped32":
            acc = torch.empty(n, dtype=torch.float32, device=dev)
            stages.append(("reduce_shard_sumsq", lambda t: F.reduce_shard_sumsq(
                grads, acc, sumsq, segs=segs_dev, n_segments=L.n_segments, workspace=ws,
                stream=stream), n * (2 * Fi + 4)))
            stages.append(("adamw_shard_step_f32grad (clipped)", lambda t: step_f32(
                acc, t, max_grad_norm=args.max_grad_norm, grad_sumsq=sumsq, **common),
                L.n_real * algorithmic_bytes_per_param_f32grad()))
        else:
            acc = torch.empty(n, dtype=torch.float32, device=dev)
            stages.append(("reduce_shard", lambda t: F.reduce_shard(grads, acc, stream=stream),
                           n * (2 * Fi + 4)))
            for mb in range(1, args.micro_batches - 1):
                stages.append((f"reduce_shard_accumulate[{mb}]", lambda t: F.reduce_shard_accumulate(
                    grads, acc, stream=stream), n * (2 * Fi + 8)))
            if args.micro_batches > 1:
                stages.append((f"reduce_shard_sumsq (accumulate)[{args.micro_batches - 1}]",
                               lambda t: F.reduce_shard_sumsq(
                                   grads, acc, sumsq, accumulate=True, segs=segs_dev,
                                   n_segments=L.n_segments, workspace=ws, stream=stream),
                               n * (2 * Fi + 8)))
            else:
                stages.append(("grad_sumsq_shard (fp32)", lambda t: F.grad_sumsq_shard(
                    sumsq, grad=acc, n=n, segs=segs_dev, n_segments=L.n_segments, workspace=ws,
                    stream=stream), n * 4))
            stages.append(("adamw_shard_step_f32grad (clipped)", lambda t: step_f32(
                acc, t, max_grad_norm=args.max_grad_norm, grad_sumsq=sumsq, **common),
                L.n_real * algorithmic_bytes_per_param_f32grad()))

    step_bytes = sum(b for _, _, b in stages)
    evict_mb = args.evict_mb if args.evict_mb >= 0 else (1024 if step_bytes < 2e9 else 0)
    evict = (torch.zeros(evict_mb << 18, dtype=torch.float32, device=dev) if evict_mb
             else None)

    def one_step(t, ev=None):
        if evict is not None:
            evict.add_(1.0)   # outside the kernel events: flushes the last-level cache
        F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
        for i, (_, launch, _) in enumerate(stages):
            if ev is not None:
                ev[i][0].record(stream)
            launch(t)
            if ev is not None:
                ev[i][1].record(stream)

    for t in range(1, args.warmup + 1):
        one_step(t)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in stages] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + 1 + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [sum(events[i][j][0].elapsed_time(events[i][j][1]) for j in range(len(stages)))
               for i in range(args.steps)]
    if evict is None:
        ms_per_step = wall / args.steps * 1e3
        timing = "wall clock over the timed steps"
    else:
        ms_per_step = sum(step_ms) / len(step_ms)
        timing = (f"sum of each step's HIP-event kernel times; {evict_mb} MiB written between "
                  "steps to flush the last-level cache")
    stage_info = []
    for j, (name, _, nbytes) in enumerate(stages):
        ms = [events[i][j][0].elapsed_time(events[i][j][1]) for i in range(args.steps)]
        avg = sum(ms) / len(ms)
        stage_info.append({"call": name, "avg_ms": round(avg, 4), "min_ms": round(min(ms), 4),
                           "median_ms": round(sorted(ms)[len(ms) // 2], 4),
                           "algorithmic_bytes": nbytes,
                           "GBps": round(nbytes / (avg / 1e3) / 1e9, 1)})
    main_stage = max(stage_info, key=lambda x: x["avg_ms"])
    avg_kernel_s = main_stage["avg_ms"] / 1e3
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; kernel avg {avg_kernel_s*1e3:.3f} ms")
    for x in stage_info:
        log(f"  {x['call']}: {x['avg_ms']:.3f} ms, {x['GBps']} GB/s")

    alg_bytes = main_stage["algorithmic_bytes"]
    achieved = alg_bytes / avg_kernel_s / 1e9
    traffic = counter_traffic(w.name) if args.path == "fused" else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic}

    # Same streams, same grid, trivial arithmetic: the ceiling of this access pattern.
    n8 = n - n % 8
    mix_ref = None
    if not args.no_copy_reference and n8 > 0 and args.path == "fused":
        out16 = flat[phase:phase + n8] if phase == 0 else torch.empty(n8, dtype=torch.int16,
                                                                        device=dev)
        def mix():
            if blocked:
                F.stream_mix_blocked(grads, state, out16, n8, stream=stream)
            else:
                F.stream_mix(grads, master, m, v, out16, n=n8, stream=stream)
        for _ in range(2):
            mix()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record(stream)
        for _ in range(reps):
            mix()
        b.record(stream)
        torch.cuda.synchronize()
        mix_ms = a.elapsed_time(b) / reps
        mix_ref = {"GBps": round(n8 * bpp / (mix_ms / 1e3) / 1e9, 1), "ms": round(mix_ms, 4),
                   "kernel": "fsdpshard_stream_mix (the step's loads and stores, no arithmetic)"}
        log(f"stream-mix reference: {mix_ref['GBps']} GB/s")
        del out16

    copy_ref = None
    if not args.no_copy_reference:
        del grads
        torch.cuda.empty_cache()
        copy_ref = copy_reference(F, torch, dev, stream)

    cpu = cpu_par = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w.name)
        log(f"cpu oracle: {cpu['value']:.3e} params/s")
        if args.cpu_procs > 0:
            cpu_par = cpu_baseline_parallel(w.name, args.cpu_procs)
            log(f"cpu oracle, {cpu_par['cores']} processes: {cpu_par['value']:.3e} params/s")

    value = L.n_real / (ms_per_step / 1e3)
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "flat_params": L.P,
            "world_size": w.world_size,
            "rank": w.rank,
            "slice_elems": n,
            "real_params": L.n_real,
            "fan_in": Fi,
            "segments": L.n_segments,
            "storage": "bf16 grads and params, fp32 master/m/v",
            "algorithmic_bytes_per_param": bpp if args.path == "fused" else None,
            # A step that re-read the bf16 parameters would move 2 more bytes per parameter
            # (28 + 2F); the fused kernel writes them from the updated fp32 master instead, so
            # the roofline above does not credit those bytes.
            "bytes_per_param_with_param_reread": bpp + 2 if args.path == "fused" else None,
            "GBps_with_param_reread": (round(L.n_real * (bpp + 2) / avg_kernel_s / 1e9, 1)
                                       if args.path == "fused" else None),
            "achieved_GBps_wall": round(sum(x["algorithmic_bytes"] for x in stage_info)
                                        / (ms_per_step / 1e3) / 1e9, 1),
            "kernel_avg_ms": round(avg_kernel_s * 1e3, 4),
            "step_ms_median": round(sorted(step_ms)[len(step_ms) // 2], 4),
            "step_ms_min": round(min(step_ms), 4),
            "timing": timing,
            "path": args.path,
            "state_layout": ("blocked: one array, 512-element blocks of master, m, v" if blocked
                             else "separate master, m, v arrays"),
            "stages": stage_info,
            "groups_per_wave": args.groups_per_wave or "default",
        },
        "roofline": roofline,
        "mix_reference": mix_ref,
        "copy_reference": copy_ref,
        "cpu_baseline": cpu,
        "cpu_baseline_parallel": cpu_par,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
