#!/usr/bin/env python3
"""Benchmark of one rank's sharded AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path PATH]
                    [--state blocked|separate] [--grads separate|interleaved]
                    [--no-extra-workloads] [--no-ceiling] [--no-copy-reference]
                    [--no-cpu-baseline]

A step is one pass of the whole hot path over the rank's slice: the host layout call
(shard_layout: flatten, floor-rule slice, segment table) and the fused GPU step
(adamw_shard_step: rank-order fp32 reduction of the F bf16 contributions, AdamW on the fp32
master / m / v, bf16 copy into the flat parameter layout).  Inputs are synthetic, seeded and
resident in HBM before the timed region; the gradient buffers are drawn once and re-read by every
step.  The timed region is K steps bracketed by device synchronisation; each kernel launch is also
bracketed by HIP events on the stream it runs on, which gives the kernel's own average duration
for the roofline figure.

The default run times the 7B-shaped slice (the headline `value`), then the memory-system
references under "ceiling", then, under "workloads", the 70B-shaped, one-layer and 2,000-tensor
slices, the separate-array entry point on the 7B-shaped slice and the 7B-shaped slice with its
contributions interleaved in one array (each of these in a fresh process of its own), then the
CPU oracle.

Prints one JSON line (the last line of stdout).
"""

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "params updated/sec per GPU (sharded AdamW step); achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
# Bytes each way of the plain copy that calibrates the hardware byte counters (every run that
# the counter summaries read launches it with exactly this size).
CALIB_COPY_BYTES = 4 << 30
DEFAULT_WORKLOAD = "dense7b_n8_rank0"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "fsdp_sharded_optimizer_layout_amd", "csrc")
KERNEL_SOURCE = [os.path.join(CSRC, "shard_step.hip"), os.path.join(CSRC, "stream_common.h")]
RESHARD_SOURCE = os.path.join(CSRC, "reshard.hip")
STEP_KERNEL = "void (anonymous namespace)::fused_step_kernel"
INTERLEAVED_STEP_KERNEL = "void (anonymous namespace)::fused_step_interleaved_kernel"
RESHARD_KERNEL = "(anonymous namespace)::reshard_kernel"
# Workloads measured after the headline in the default run: (name, layout).  Layouts: "blocked"
# (blocked state, F separate contributions), "separate" (three state arrays, F contributions),
# "interleaved" (blocked state, the F contributions interleaved per block in one array).
EXTRA_WORKLOADS = [("dense70b_n64_rank0", "blocked"), ("llama_layer_n8_rank0", "blocked"),
                   ("many_small_n16_rank3", "blocked"), ("dense7b_n8_rank0", "separate"),
                   ("dense7b_n8_rank0", "interleaved")]
LAYOUT_DESCRIPTION = {
    "blocked": "blocked: one array, 512-element blocks of master, m, v",
    "separate": "separate master, m, v arrays",
    "interleaved": ("blocked state; the F contributions interleaved per 512-element block in "
                    "one array"),
}


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
    """Digest of kernel sources (a path or a list of paths) with comments and whitespace removed:
    the counter figures stay valid across comment edits and lapse with any change to the code."""
    import re
    paths = [source] if isinstance(source, str) else list(source)
    text = ""
    for path in paths:
        with open(path) as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def traffic_key(workload, layout="blocked"):
    return workload if layout == "blocked" else f"{workload}:{layout}"


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
                       calib_kernel="stream_copy_kernel", calib_bytes=None):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch) into per-launch HBM bytes of the measured kernel, each counter scaled by what it
    reads for the plain copy kernel, whose true traffic is calib_bytes read and calib_bytes
    written.  Writes the result into profiles/traffic.json under `key`."""
    import csv
    import statistics
    if calib_bytes is None:
        calib_bytes = CALIB_COPY_BYTES

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


# ----------------------------------------------------------------------------- CPU oracle baseline

def host_cores():
    """What the host offers this process: os.cpu_count(), the CPUs in its affinity mask, and the
    cgroup CPU quota (cpu.max) if one is set.  `usable` is the smaller of the last two."""
    n_os = os.cpu_count()
    aff = len(os.sched_getaffinity(0))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
        if q != "max":
            quota = max(1, math.ceil(int(q) / int(period)))
    except (OSError, ValueError):
        pass
    return {"os_cpu_count": n_os, "affinity": aff, "cgroup_quota": quota,
            "usable": min(aff, quota) if quota else aff}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_inputs(workload, a, b):
    """Flags, initial state and one step's contributions for elements [a, b) of the slice."""
    import numpy as np
    import workloads as W
    from oracle import layout as OL

    w = W.WORKLOADS[workload]
    lo, hi, osegs = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    flags = np.zeros(b - a, dtype=np.int64)
    for s in osegs:
        x, y = max(a, s["shard_begin"]), min(b, s["shard_begin"] + s["length"])
        if x < y:
            flags[x - a:y - a] = s["flags"]
    master, m, v = W.np_state(w, b - a, a)
    grads = W.np_grads(w, b - a, 1, a)
    n_real = int(np.count_nonzero((flags & OL.PADDING) == 0))
    return w, flags, master, m, v, grads, n_real


def _oracle_steps(w, flags, master, m, v, grads, seconds):
    """Oracle steps on one chunk until `seconds` have passed; returns (steps, elapsed)."""
    from oracle import step as OS
    steps = 0
    t0 = time.perf_counter()
    while True:
        steps += 1
        master, m, v, _ = OS.shard_step(master, m, v, grads, flags, w.hp, steps)
        el = time.perf_counter() - t0
        if el >= seconds:
            return steps, el


def cpu_baseline_single(workload, seconds=12.0, sample=1 << 26):
    """The oracle as it is, single-threaded NumPy, on the first `sample` elements of the same
    workload's slice (64 Mi elements: a working set far beyond the host's caches)."""
    from oracle import layout as OL
    import workloads as W

    w0 = W.WORKLOADS[workload]
    lo, hi, _ = OL.segments(w0.sizes, w0.pad_multiple, w0.wd_mask, w0.world_size, w0.rank)
    n = min(sample, hi - lo)
    w, flags, master, m, v, grads, n_real = _oracle_inputs(workload, 0, n)
    steps, el = _oracle_steps(w, flags, master, m, v, grads, seconds)
    return {"value": n_real * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"first {n} elements of the {workload} slice, fan-in {w.fan_in}, "
                      f"{steps} oracle steps in {el:.1f} s (NumPy float32, one thread)"}


def _oracle_worker(args):
    workload, a, b, seconds, barrier, results = args
    w, flags, master, m, v, grads, n_real = _oracle_inputs(workload, a, b)
    barrier.wait(timeout=600)          # every worker starts stepping at the same moment
    steps, el = _oracle_steps(w, flags, master, m, v, grads, seconds)
    results.put((n_real * steps, el))


def cpu_baseline(workload, procs, seconds=12.0, chunk=1 << 22):
    """The same oracle in `procs` processes, each stepping its own contiguous 4 Mi-element chunk
    of the slice (valid because the step is elementwise once the layout is fixed).  The workers
    draw their inputs, meet at a barrier, then step for `seconds`; rate = all workers' real
    parameters x steps / the longest worker's stepping time.  None if a worker fails."""
    import multiprocessing as mp

    import workloads as W
    from oracle import layout as OL

    w = W.WORKLOADS[workload]
    lo, hi, _ = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    n = hi - lo
    procs = max(1, min(procs, n // chunk if n >= chunk else 1))
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(procs), ctx.Queue()
    workers = [ctx.Process(target=_oracle_worker,
                           args=((workload, i * chunk, min(n, (i + 1) * chunk), seconds, barrier,
                                  results),))
               for i in range(procs)]
    for p in workers:
        p.start()
    import queue
    try:
        done = [results.get(timeout=seconds + 900) for _ in workers]
    except queue.Empty:                # a worker died: no parallel figure rather than a hang
        for p in workers:
            p.terminate()
        return None
    for p in workers:
        p.join()
    total = sum(d[0] for d in done)
    el = max(d[1] for d in done)
    cores = host_cores()
    return {"value": total / el, "unit": "params/s", "cores": procs, "kind": "oracle",
            "cpu": cpu_model(), "host": cores,
            "sample": f"{procs} processes (one per usable host core: {cores['affinity']} CPUs in "
                      f"the affinity mask, cgroup quota {cores['cgroup_quota']}, os.cpu_count() "
                      f"{cores['os_cpu_count']}), each stepping the oracle on its own "
                      f"{chunk}-element chunk of the {workload} slice for {seconds:.0f} s "
                      f"(NumPy float32, one thread each)"}


# ----------------------------------------------------------------------------- GPU measurement

class Slice:
    """Device buffers of one workload's slice: state (blocked or separate), F contributions (and
    with the interleaved layout their interleaved copy), the bf16 flat window and the segment
    table.  `layout` is one of LAYOUT_DESCRIPTION's keys (True / False mean blocked /
    separate)."""

    def __init__(self, F, W, torch, name, layout, dev):
        layout = {True: "blocked", False: "separate"}.get(layout, layout)
        blocked = layout != "separate"
        w = W.WORKLOADS[name]
        self.w, self.layout, self.blocked, self.dev = w, layout, blocked, dev
        self.L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
        n, lo = self.L.n, self.L.lo
        master, m, v = W.torch_state(w, n, 0, dev)
        self.grads = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(w.fan_in)]
        W.torch_grads_into(w, self.grads, 1, 0)
        if w.nan_padding_grads:
            for s in segs:
                if s["flags"] & F.SEG_PADDING:
                    for g in self.grads:
                        g[int(s["shard_begin"]): int(s["shard_begin"] + s["length"])] = 0x7FC0
        self.gi = None
        if layout == "interleaved":
            self.gi = torch.empty(F.grads_interleaved_elems(w.fan_in, n), dtype=torch.int16,
                                  device=dev)
            F.grads_to_interleaved(self.grads, self.gi, n=n)
        self.phase = lo % 8
        self.flat = torch.empty(n + self.phase, dtype=torch.int16, device=dev)
        self.segs_dev = F.segments_to_device(segs, dev)
        if blocked:
            self.state = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device=dev)
            F.state_to_blocked(master, m, v, self.state)
            torch.cuda.synchronize()
            del master, m, v
            self.master = self.m = self.v = None
        else:
            self.state = None
            self.master, self.m, self.v = master, m, v
        torch.cuda.synchronize()

    def common(self, stream):
        L = self.L
        return dict(segs=self.segs_dev, n_segments=L.n_segments, flat=self.flat,
                    flat_index0=L.lo - self.phase, lo=L.lo, stream=stream, **self.w.hp)

    def step_bf16(self, F, t, **kw):
        if self.gi is not None:
            F.adamw_shard_step_interleaved(self.state, self.gi, self.w.fan_in, step=t,
                                           n=self.L.n, **kw)
        elif self.blocked:
            F.adamw_shard_step_blocked(self.state, self.grads, step=t, n=self.L.n, **kw)
        else:
            F.adamw_shard_step(self.master, self.m, self.v, self.grads, step=t, **kw)

    def step_f32(self, F, acc, t, **kw):
        if self.blocked:
            F.adamw_shard_step_f32grad_blocked(self.state, acc, step=t, n=self.L.n, **kw)
        else:
            F.adamw_shard_step_f32grad(self.master, self.m, self.v, acc, step=t, **kw)


def build_stages(F, torch, S, path, stream, args):
    """Stages of one step: (name, launch(t), algorithmic bytes per launch)."""
    L, n, Fi, dev = S.L, S.L.n, S.w.fan_in, S.dev
    bpp = algorithmic_bytes_per_param(Fi)
    common = S.common(stream)
    stages = []
    suffix = {"blocked": "_blocked", "separate": "", "interleaved": "_interleaved"}[S.layout]
    f32_suffix = "" if S.layout == "separate" else "_blocked"
    il = S.gi is not None
    if il and path == "split":
        raise ValueError("the split path reads separate contributions")
    if path == "fused":
        stages.append(("adamw_shard_step" + suffix, lambda t: S.step_bf16(F, t, **common),
                       L.n_real * bpp))
    elif path == "split":
        no_out = {k: v for k, v in common.items() if k not in ("flat", "flat_index0", "lo")}
        stages.append(("adamw_shard_step (no bf16 output)", lambda t: F.adamw_shard_step(
            S.master, S.m, S.v, S.grads, step=t, **no_out), L.n_real * (bpp - 2)))
        stages.append(("unflatten_bf16", lambda t: F.unflatten_bf16(
            S.master, S.flat, flat_index0=L.lo - S.phase, lo=L.lo, segs=S.segs_dev,
            n_segments=L.n_segments, stream=stream), L.n_real * 4 + n * 2))
    else:
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        ws = torch.empty(max(8, F.grad_sumsq_workspace_bytes(n)), dtype=torch.uint8, device=dev)
        segkw = dict(segs=S.segs_dev, n_segments=L.n_segments, workspace=ws, stream=stream)
        clip = dict(max_grad_norm=args.max_grad_norm, grad_sumsq=sumsq)
        f32_bytes = L.n_real * algorithmic_bytes_per_param_f32grad()
        # The contributions' calls: from F arrays, or from the interleaved array.
        if il:
            sumsq_bf16 = lambda: F.grad_sumsq_shard_interleaved(sumsq, S.gi, Fi, n, **segkw)
            red = lambda acc, a: F.reduce_shard_interleaved(S.gi, Fi, acc, accumulate=a,
                                                            stream=stream)
            red_sq = lambda acc, a: F.reduce_shard_sumsq_interleaved(S.gi, Fi, acc, sumsq,
                                                                     accumulate=a, **segkw)
        else:
            sumsq_bf16 = lambda: F.grad_sumsq_shard(sumsq, contribs=S.grads, n=n, **segkw)
            red = lambda acc, a: (F.reduce_shard_accumulate(S.grads, acc, stream=stream) if a
                                  else F.reduce_shard(S.grads, acc, stream=stream))
            red_sq = lambda acc, a: F.reduce_shard_sumsq(S.grads, acc, sumsq, accumulate=a,
                                                         **segkw)
        isfx = "_interleaved" if il else ""
        if path == "clipped":
            stages.append(("grad_sumsq_shard" + isfx, lambda t: sumsq_bf16(), n * 2 * Fi))
            stages.append(("adamw_shard_step" + suffix + " (clipped)", lambda t: S.step_bf16(
                F, t, **clip, **common), L.n_real * bpp))
        elif path == "clipped32":
            acc = torch.empty(n, dtype=torch.float32, device=dev)
            stages.append(("reduce_shard_sumsq" + isfx, lambda t: red_sq(acc, False),
                           n * (2 * Fi + 4)))
            stages.append(("adamw_shard_step_f32grad" + f32_suffix + " (clipped)",
                           lambda t: S.step_f32(F, acc, t, **clip, **common), f32_bytes))
        else:   # accumulate
            acc = torch.empty(n, dtype=torch.float32, device=dev)
            stages.append(("reduce_shard" + isfx, lambda t: red(acc, False), n * (2 * Fi + 4)))
            for mb in range(1, args.micro_batches - 1):
                name = "reduce_shard_interleaved (accumulate)" if il else "reduce_shard_accumulate"
                stages.append((f"{name}[{mb}]", lambda t: red(acc, True), n * (2 * Fi + 8)))
            if args.micro_batches > 1:
                stages.append((f"reduce_shard_sumsq{isfx} (accumulate)[{args.micro_batches - 1}]",
                               lambda t: red_sq(acc, True), n * (2 * Fi + 8)))
            else:
                stages.append(("grad_sumsq_shard (fp32)", lambda t: F.grad_sumsq_shard(
                    sumsq, grad=acc, n=n, **segkw), n * 4))
            stages.append(("adamw_shard_step_f32grad" + f32_suffix + " (clipped)",
                           lambda t: S.step_f32(F, acc, t, **clip, **common), f32_bytes))
    return stages


def make_evict(torch, dev, step_bytes, evict_mb):
    """A 1 GiB buffer written between timed steps of workloads that move under 2 GB per step, so
    the 256 MB last-level cache holds none of the step's data when the next one starts."""
    mb = evict_mb if evict_mb >= 0 else (1024 if step_bytes < 2e9 else 0)
    return mb, (torch.zeros(mb << 18, dtype=torch.float32, device=dev) if mb else None)


def time_stages(F, torch, S, stages, stream, steps, warmup, evict):
    """W warm-up steps, then `steps` timed steps (host layout call + every stage), each stage
    bracketed by HIP events on `stream`."""
    w = S.w

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

    for t in range(1, warmup + 1):
        one_step(t)
    torch.cuda.synchronize()
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in stages] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(warmup + 1 + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [sum(events[i][j][0].elapsed_time(events[i][j][1]) for j in range(len(stages)))
               for i in range(steps)]
    if evict is None:
        ms_per_step = wall / steps * 1e3
        timing = "wall clock over the timed steps"
    else:
        ms_per_step = sum(step_ms) / len(step_ms)
        timing = (f"sum of each step's HIP-event kernel times; {evict.numel() >> 18} MiB written "
                  "between steps to flush the last-level cache")
    info = []
    for j, (name, _, nbytes) in enumerate(stages):
        ms = [events[i][j][0].elapsed_time(events[i][j][1]) for i in range(steps)]
        avg = sum(ms) / len(ms)
        info.append({"call": name, "avg_ms": round(avg, 4), "min_ms": round(min(ms), 4),
                     "median_ms": round(sorted(ms)[len(ms) // 2], 4),
                     "algorithmic_bytes": nbytes, "GBps": round(nbytes / (avg / 1e3) / 1e9, 1)})
    return {"ms_per_step": ms_per_step, "step_ms": step_ms, "stages": info, "timing": timing}


def time_launches(torch, launch, stream, reps=5, warm=2, evict=None):
    """Average HIP-event time of `launch` (per launch when a flush runs between launches)."""
    for _ in range(warm):
        launch()
    torch.cuda.synchronize()
    if evict is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    total = 0.0
    for _ in range(reps):
        evict.add_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b.record(stream)
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
    return total / reps


# Launch shapes of the step's traffic replica (groups per wave, work-groups per CU, XCD run,
# phased): the step's own shape, the best unphased shapes of a sweep of the exact bytes at
# fan-in 8, and phased shapes (each work-group's loads before any of its stores).
MIX_SHAPES = [(1, 2, 32, 0), (1, 1, 16, 0), (1, 1, 64, 0), (1, 2, 32, 1), (2, 1, 32, 1),
              (4, 1, 32, 1)]


def mix_references(F, torch, S, stream, evict, shapes=False):
    """The step's loads and stores with trivial arithmetic on this slice's own buffers: in the
    step's order (same grid, tile map and work-groups per CU), and, with `shapes`, in the other
    launch shapes of MIX_SHAPES (blocked state only); `best` is the fastest of them."""
    n8 = S.L.n - S.L.n % 8
    if n8 == 0:
        return None
    bpp = algorithmic_bytes_per_param(S.w.fan_in)
    out16 = (S.flat[S.phase:S.phase + n8] if S.phase == 0
             else torch.empty(n8, dtype=torch.int16, device=S.dev))
    if S.gi is not None:
        mix = lambda: F.stream_mix_interleaved(S.gi, S.w.fan_in, S.state, out16, n8,
                                               stream=stream)
    elif S.blocked:
        mix = lambda: F.stream_mix_blocked(S.grads, S.state, out16, n8, stream=stream)
    else:
        mix = lambda: F.stream_mix(S.grads, S.master, S.m, S.v, out16, n=n8, stream=stream)
    ms = time_launches(torch, mix, stream, evict=evict)
    suffix = {"blocked": "_blocked", "separate": "", "interleaved": "_interleaved"}[S.layout]
    ref = {"step_order": {"GBps": round(n8 * bpp / (ms / 1e3) / 1e9, 1), "ms": round(ms, 4),
                          "kernel": "fsdpshard_stream_mix" + suffix},
           "flushed": evict is not None}
    best = dict(ref["step_order"], shape="the step's")
    if shapes and S.layout == "blocked" and S.w.fan_in in (1, 4, 8):
        for G, per_cu, run, phased in MIX_SHAPES:
            ms = time_launches(torch, lambda: F.stream_mix_shaped(
                S.grads, S.state, out16, n8, G, per_cu, run, phased, stream=stream), stream,
                evict=evict)
            name = f"g{G}_cu{per_cu}_run{run}" + ("_phased" if phased else "")
            ref[name] = {"GBps": round(n8 * bpp / (ms / 1e3) / 1e9, 1), "ms": round(ms, 4)}
            if ref[name]["GBps"] > best["GBps"]:
                best = dict(ref[name], shape=name)
    ref["best"] = best
    del out16
    return ref


def f32_step_reference(F, torch, S, stream, evict):
    """The fp32-gradient step's bytes with trivial arithmetic (blocked state): the interleaved
    replica at fan-in 2 reads 4 bytes of gradient per element, 2 KiB contiguous per 512-element
    block, as the step reads its fp32 shard; with 24 bytes of state and the 2-byte bf16 copy it
    moves the step's 30 bytes per element, in the step's grid, tile map and work-groups per CU."""
    n8 = S.L.n - S.L.n % 8
    if n8 == 0 or not S.blocked:
        return None
    g2 = torch.zeros(F.grads_interleaved_elems(2, n8), dtype=torch.int16, device=S.dev)
    out16 = (S.flat[S.phase:S.phase + n8] if S.phase == 0
             else torch.empty(n8, dtype=torch.int16, device=S.dev))
    ms = time_launches(torch, lambda: F.stream_mix_interleaved(g2, 2, S.state, out16, n8,
                                                               stream=stream),
                       stream, evict=evict)
    bpe = algorithmic_bytes_per_param_f32grad()
    del g2, out16
    return {"f32grad_step_bytes": {"GBps": round(n8 * bpe / (ms / 1e3) / 1e9, 1),
                                   "ms": round(ms, 4),
                                   "kernel": "fsdpshard_stream_mix_interleaved (fan-in 2)"},
            "flushed": evict is not None}


def measure_workload(F, W, torch, name, layout, args, dev, stream, mix=True):
    """The fused step of one workload: its stage timing, roofline figures and (like for like,
    flushed when the step is) the traffic replica."""
    S = Slice(F, W, torch, name, layout, dev)
    stages = build_stages(F, torch, S, "fused", stream, args)
    evict_mb, evict = make_evict(torch, dev, stages[0][2], args.evict_mb)
    r = time_stages(F, torch, S, stages, stream, args.steps, args.warmup, evict)
    st = r["stages"][0]
    bpp = algorithmic_bytes_per_param(S.w.fan_in)
    gbps = st["algorithmic_bytes"] / (st["avg_ms"] / 1e3) / 1e9
    out = {"workload": name, "layout": layout,
           "state_layout": LAYOUT_DESCRIPTION[layout],
           "call": st["call"], "fan_in": S.w.fan_in, "slice_elems": S.L.n,
           "real_params": S.L.n_real, "segments": S.L.n_segments, "dest_phase": S.phase,
           "algorithmic_bytes_per_param": bpp,
           "kernel_avg_ms": st["avg_ms"], "kernel_min_ms": st["min_ms"],
           "ms_per_step": round(r["ms_per_step"], 4),
           "params_per_s": round(S.L.n_real / (r["ms_per_step"] / 1e3), 1),
           "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
           "traffic": counter_traffic(traffic_key(name, layout)),
           "timing": r["timing"]}
    if mix and not args.no_copy_reference:
        out["mix_reference"] = mix_references(F, torch, S, stream, evict)
    del S, evict
    torch.cuda.empty_cache()
    return out


# Launch shapes of the plain-stream probes (vectors per thread, threads per work-group,
# work-groups per CU, XCD run): the fastest few of a sweep of 216 shapes per stream kind on
# MI355X.
CEILING_SHAPES = {
    "read": [(1, 1024, 0, 1), (4, 1024, 0, 32), (2, 512, 0, 32)],
    "write": [(2, 256, 2, 256), (1, 256, 4, 1), (2, 256, 2, 32)],
    "copy": [(2, 256, 0, 256), (1, 256, 0, 1), (2, 1024, 0, 32)],
    "read2_write1": [(1, 256, 0, 256), (2, 512, 0, 32), (1, 256, 0, 32)],
}
# Streams read and written in place (as the step's state) take the shapes of their out-of-place
# counterparts; eight read streams (the step's gradient count) the shapes that did best for them.
CEILING_SHAPES["inplace"] = CEILING_SHAPES["copy"]
CEILING_SHAPES["read1_inplace1"] = CEILING_SHAPES["read2_write1"]
CEILING_SHAPES["read8"] = [(1, 256, 0, 32), (1, 256, 0, 256), (2, 512, 0, 32)]
CEILING_SHAPES["read8_write1"] = [(1, 256, 0, 1), (1, 256, 0, 32), (2, 512, 0, 32)]
CEILING_SHAPES["read7_inplace1"] = CEILING_SHAPES["read8_write1"]


def ceiling_references(F, torch, dev, stream, read_bytes, write_bytes, nbytes=2 << 30):
    """What the memory system does for plain streams on this GPU, each the best of a few launch
    shapes: pure reads and pure writes, a copy, the step's 2 : 1 read : write byte ratio, each
    also with its written stream read and written in place as the step's state is, and eight
    read streams (the step's gradient streams at fan-in 8) alone, into one write stream and with
    one of them written in place; plus the time bound the pure rates imply for the step's
    bytes."""
    # One allocation cut into nine streams.
    n4 = nbytes // 4
    whole = torch.ones(9 * n4, dtype=torch.float32, device=dev)
    bufs = [whole[i * n4:(i + 1) * n4] for i in range(9)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    A, B, C = bufs[:3]
    cases = {"read": ([A, B], []), "write": ([], [A, B]), "copy": ([A], [B]),
             "read2_write1": ([A, B], [C]), "inplace": ([A], [A]), "read1_inplace1": ([A, B], [B]),
             "read8": (bufs[:8], []), "read8_write1": (bufs[:8], [bufs[8]]),
             "read7_inplace1": (bufs[:8], [bufs[7]])}
    out = {}
    for name, (srcs, dsts) in cases.items():
        moved = (len(srcs) + len(dsts)) * nbytes
        best = None
        for vpt, threads, per_cu, run in CEILING_SHAPES[name]:
            ms = time_launches(torch, lambda: F.stream_rw(
                srcs, dsts, nbytes, vectors_per_thread=vpt, threads_per_group=threads,
                per_cu=per_cu, xcd_run=run, sink=sink, stream=stream), stream, reps=10)
            gbps = moved / (ms / 1e3) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": round(gbps, 1), "shape": [vpt, threads, per_cu, run]}
        out[name] = best
        log(f"  {name}: {best['GBps']} GB/s (vectors per thread, threads, per CU, XCD run: "
            f"{best['shape']})")
    # If a channel could only read at the pure-read rate and write at the pure-write rate, one
    # after the other, the step's bytes would need at least this long.
    t = read_bytes / (out["read"]["GBps"] * 1e9) + write_bytes / (out["write"]["GBps"] * 1e9)
    out["serial_rw_bound"] = {
        "GBps": round((read_bytes + write_bytes) / t / 1e9, 1),
        "read_bytes": read_bytes, "write_bytes": write_bytes,
        "meaning": "the step's read and write bytes at the pure-read and pure-write rates, one "
                   "after the other"}
    del bufs, A, B, C, sink, whole
    torch.cuda.empty_cache()
    return out


def run_child(args, spec):
    """One measurement (`--child spec`) in a fresh Python process on the same GPU; its record, or
    {"error": ...} if the child failed (the headline line is printed either way)."""
    cmd = [sys.executable, os.path.abspath(__file__), "--child", spec, "--workload", args.workload,
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--evict-mb",
           str(args.evict_mb)]
    if args.no_copy_reference:
        cmd.append("--no-copy-reference")
    try:
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900)
    except subprocess.TimeoutExpired:
        log(f"measurement {spec} timed out")
        return {"error": "timed out"}
    if r.returncode != 0:
        log(f"measurement {spec} failed with status {r.returncode}")
        return {"error": f"exit status {r.returncode}"}
    return json.loads(r.stdout.strip().splitlines()[-1])


def child_measurement(args, w, F, W, torch, dev, stream):
    """The measurement `args.child` names, in this (fresh) process."""
    if args.child == "ceiling":
        L, _ = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
        return ceiling_references(F, torch, dev, stream, L.n_real * (2 * w.fan_in + 12),
                                  L.n_real * 14)
    kind, name, layout = args.child.split(":")
    if kind != "workload" or layout not in LAYOUT_DESCRIPTION:
        raise ValueError(f"unknown measurement {args.child}")
    return measure_workload(F, W, torch, name, layout, args, dev, stream)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--path", choices=["fused", "clipped", "clipped32", "accumulate", "split",
                                       "reshard"],
                    default="fused",
                    help="fused: the fused step (default); clipped: sum of squares + clipped "
                         "step; clipped32: reduction fused with the sum of squares into an fp32 "
                         "shard + clipped fp32-gradient step; accumulate: fp32 micro-batch "
                         "accumulation (the last fused with the sum of squares) + clipped fp32 "
                         "step; split: the step without its bf16 output, then unflatten_bf16; "
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
    ap.add_argument("--grads", choices=["separate", "interleaved"], default="separate",
                    help="gradient contributions: F separate arrays (default), or interleaved per "
                         "512-element block in one array (blocked state only)")
    ap.add_argument("--max-grad-norm", type=float, default=1.0)
    ap.add_argument("--evict-mb", type=int, default=-1,
                    help="MiB written between timed steps to flush the 256 MB last-level cache "
                         "(-1: 1024 when one step moves under 2 GB, else 0); with eviction the "
                         "per-step time is the sum of the step's HIP-event kernel times")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="processes for the parallel oracle baseline (0: one per usable host "
                         "core; -1: skip it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-reference", action="store_true",
                    help="skip the traffic replicas and the memory-system references")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="time only the selected workload")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the memory-system references (the plain copy that calibrates the "
                         "hardware counters still runs)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    # One measurement of the default run in a process of its own: "ceiling", or
    # "workload:NAME:LAYOUT".  Prints its JSON record as the last line of stdout.
    ap.add_argument("--child", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.summarize_counters:
        if args.path == "reshard":
            import workloads as W
            w = W.WORKLOADS[args.workload]
            key = reshard_key(w.name, args.reshard_world, args.reshard_pad or w.pad_multiple,
                              args.reshard_rank)
            summarize_counters(key, *args.summarize_counters, kernel_prefix=RESHARD_KERNEL,
                               source=RESHARD_SOURCE)
        elif args.grads == "interleaved":
            summarize_counters(traffic_key(args.workload, "interleaved"),
                               *args.summarize_counters, kernel_prefix=INTERLEAVED_STEP_KERNEL)
        else:
            summarize_counters(traffic_key(args.workload, args.state),
                               *args.summarize_counters)
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

    w = W.WORKLOADS[args.workload]
    if args.path == "reshard":
        bench_reshard(args, w, F, W, torch)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.child:
        print(json.dumps(child_measurement(args, w, F, W, torch, dev, stream)), flush=True)
        return
    blocked = args.state == "blocked" and args.path != "split"
    if args.grads == "interleaved" and not blocked:
        print("--grads interleaved needs the blocked state (and not the split path)",
              file=sys.stderr)
        sys.exit(2)
    layout = ("interleaved" if args.grads == "interleaved" else "blocked") if blocked else "separate"
    S = Slice(F, W, torch, w.name, layout, dev)
    L, Fi = S.L, w.fan_in
    log(f"workload {w.name}: P={L.P} slice [{L.lo}, {L.hi}) n={L.n} n_real={L.n_real} "
        f"F={Fi} segments={L.n_segments}")
    bpp = algorithmic_bytes_per_param(Fi)
    stages = build_stages(F, torch, S, args.path, stream, args)
    step_bytes = sum(b for _, _, b in stages)
    evict_mb, evict = make_evict(torch, dev, step_bytes, args.evict_mb)
    r = time_stages(F, torch, S, stages, stream, args.steps, args.warmup, evict)
    ms_per_step, stage_info = r["ms_per_step"], r["stages"]
    main_stage = max(stage_info, key=lambda x: x["avg_ms"])
    avg_kernel_s = main_stage["avg_ms"] / 1e3
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; kernel avg "
        f"{avg_kernel_s * 1e3:.3f} ms")
    for x in stage_info:
        log(f"  {x['call']}: {x['avg_ms']:.3f} ms, {x['GBps']} GB/s")
    achieved = main_stage["algorithmic_bytes"] / avg_kernel_s / 1e9
    traffic = counter_traffic(traffic_key(w.name, layout)) if args.path == "fused" else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic}

    mix_ref = None
    if not args.no_copy_reference and args.path == "fused":
        mix_ref = mix_references(F, torch, S, stream, evict, shapes=True)
        for k, x in (mix_ref or {}).items():
            if isinstance(x, dict):
                log(f"  traffic replica {k}: {x['GBps']} GB/s")
    elif not args.no_copy_reference and args.path in ("clipped32", "accumulate"):
        # These paths end with the fp32-gradient step: replay its bytes on the same buffers.
        mix_ref = f32_step_reference(F, torch, S, stream, evict)
        if mix_ref:
            log(f"  fp32-gradient step replica: {mix_ref['f32grad_step_bytes']['GBps']} GB/s")
    del S, stages, evict
    torch.cuda.empty_cache()

    # The memory-system references and every other workload run in a fresh process each: the
    # bandwidth of a set of buffers depends on where in memory they land, and that depends on
    # what the process allocated and freed before (measured on one box: the 2 : 1 reference
    # read 4 % lower after the other workloads' allocations, and the separate-array step 7 %
    # lower after the references').  A fresh process sees what a run of that workload alone
    # sees.
    ceiling = None
    if not args.no_copy_reference:
        # The counters' calibration copy runs in this process, beside the measured kernel.
        calib = copy_reference(F, torch, dev, stream)
        torch.cuda.empty_cache()
        ceiling = {}
        if not args.no_ceiling:
            log("memory-system references:")
            ceiling = run_child(args, "ceiling")
        ceiling["copy_plain"] = dict(calib, kernel="fsdpshard_stream_copy (the counters' "
                                                   "calibration kernel)")

    extra = None
    if args.path == "fused" and not args.no_extra_workloads:
        extra = []
        for name, lay in EXTRA_WORKLOADS:
            if name == w.name and lay == layout:
                continue
            x = run_child(args, f"workload:{name}:{lay}")
            if "error" in x:
                x = dict(x, workload=name, layout=lay)
            else:
                log(f"workload {name} ({x['state_layout']}): {x['kernel_avg_ms']:.4f} ms, "
                    f"{x['GBps']} GB/s, frac {x['frac']}")
            extra.append(x)

    cpu = cpu_single = None
    if not args.no_cpu_baseline:
        cores = host_cores()
        procs = args.cpu_procs if args.cpu_procs > 0 else cores["usable"]
        log(f"timing the CPU oracle (host cores {cores}) ...")
        cpu_single = cpu_baseline_single(w.name)
        log(f"cpu oracle, one thread: {cpu_single['value']:.3e} params/s")
        if args.cpu_procs >= 0:
            cpu = cpu_baseline(w.name, procs)
            if cpu is None:
                log("cpu oracle: a worker process failed; reporting the one-thread figure")
            else:
                log(f"cpu oracle, {cpu['cores']} processes: {cpu['value']:.3e} params/s")
        if cpu is None:
            cpu = cpu_single

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
            "slice_elems": L.n,
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
            "step_ms_median": round(sorted(r["step_ms"])[len(r["step_ms"]) // 2], 4),
            "step_ms_min": round(min(r["step_ms"]), 4),
            "timing": r["timing"],
            "path": args.path,
            "state_layout": LAYOUT_DESCRIPTION[layout],
            "stages": stage_info,
        },
        "roofline": roofline,
        "workloads": extra,
        "mix_reference": mix_ref,
        "ceiling": ceiling,
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu_single,
    }
    print(json.dumps(rec), flush=True)


# ----------------------------------------------------------------------------- reshard path

def copy_reference(F, torch, dev, stream, nbytes=None):
    """Plain 16-byte copy of nbytes (non-temporal loads and stores): the bandwidth a pure
    read+write stream reaches, and the calibration kernel of the counter runs."""
    if nbytes is None:
        nbytes = CALIB_COPY_BYTES
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms = time_launches(torch, lambda: F.stream_copy(src, dst, stream=stream), stream, reps=10,
                       warm=3)
    ref = {"GBps": round(2 * nbytes / (ms / 1e3) / 1e9, 1), "bytes_moved": 2 * nbytes,
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



if __name__ == "__main__":
    main()
