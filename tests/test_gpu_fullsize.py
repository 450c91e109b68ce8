"""Full-size parity: each shard configuration at its real shape, in the launch configuration the
benchmark times, compared with the oracle on sampled windows of the slice.

The step is elementwise once the layout is fixed, so the oracle can recompute any subset of
elements from the same inputs.  Windows: the first and last 1 Mi elements, +-4 Ki around every
segment edge inside the slice, and 64 random 64 Ki windows.  Inputs are drawn on the device with
seeded generators (no value comes from the library); the oracle receives copies of exactly the
windowed inputs.  The bf16 destination uses the phase the slice has in a 16-byte aligned flat
vector (lo mod 8), and a guarded prefix / suffix of the flat window must survive.  Each workload
runs its full step count, through the separate-array entry point and through the blocked-state
one the benchmark times; besides the tolerance bars (fp32 relative 1e-5, bf16 1 ulp) every
sampled value must equal the oracle's bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from oracle import clip as OC
from oracle import layout as OL
from oracle import step as OS
import blocked_layout as BL
from gpu_helpers import SENT16, assert_bf16, assert_f32, bit_equal, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
WIN = 65536
END = 1 << 20
EDGE = 4096


def _windows(n, edges, rng):
    spans = [(0, END), (n - END, n)] + [(e - EDGE, e + EDGE) for e in edges]
    for s in rng.integers(0, max(1, n - WIN), 64):
        spans.append((int(s), int(s) + WIN))
    mask_idx = []
    for a, b in spans:
        a, b = max(0, a), min(n, b)
        if a < b:
            mask_idx.append(np.arange(a, b, dtype=np.int64))
    return np.unique(np.concatenate(mask_idx))


def _flags_at(osegs, idx):
    starts = np.array([s["shard_begin"] for s in osegs], dtype=np.int64)
    fl = np.array([s["flags"] for s in osegs], dtype=np.int64)
    return fl[np.searchsorted(starts, idx, side="right") - 1]


def _blocked_index(idx, k):
    """Position of element idx's k-th state value (0 master, 1 m, 2 v) in the blocked array."""
    return ((idx // BL.STATE_BLOCK) * 3 + k) * BL.STATE_BLOCK + idx % BL.STATE_BLOCK


def _check(got, want, what, exact=True):
    if want.dtype == np.uint16:
        assert_bf16(got, want, what)
    else:
        assert_f32(got, want, what)
    if exact:
        assert bit_equal(got, want), f"{what}: not bit-equal to the oracle"


def run_fullsize(name, blocked, seed=0):
    w = W.WORKLOADS[name]
    L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    lo_o, hi_o, osegs = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    assert (L.lo, L.hi) == (lo_o, hi_o)
    n, lo = L.n, L.lo
    say(f"fullsize {name} ({'blocked' if blocked else 'separate'} state): n={n} lo={lo} "
        f"F={w.fan_in} segs={L.n_segments}")
    edges = [s["shard_begin"] for s in osegs[1:]]
    rng = np.random.default_rng(seed)
    idx = _windows(n, edges, rng)
    idx_t = torch.from_numpy(idx).cuda()
    flags = _flags_at(osegs, idx)
    pad_mask_dev = None
    if w.nan_padding_grads:
        pad_mask_dev = torch.zeros(n, dtype=torch.bool, device="cuda")
        for s in osegs:
            if s["flags"] & OL.PADDING:
                pad_mask_dev[s["shard_begin"]: s["shard_begin"] + s["length"]] = True

    master, m, v = W.torch_state(w, n, seed, "cuda")
    om = master[idx_t].cpu().numpy()
    omm = m[idx_t].cpu().numpy()
    ov = v[idx_t].cpu().numpy()
    if blocked:
        state = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device="cuda")
        F.state_to_blocked(master, m, v, state)
        torch.cuda.synchronize()
        del master, m, v
        pos = [torch.from_numpy(_blocked_index(idx, k)).cuda() for k in range(3)]
        read = [lambda k=k: state[pos[k]].cpu().numpy() for k in range(3)]
    else:
        read = [lambda x=x: x[idx_t].cpu().numpy() for x in (master, m, v)]
    grads = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(w.fan_in)]
    phase = lo % 8
    GUARD = 64
    flat_full = torch.full((GUARD + phase + n + GUARD,), int(SENT16),
                           dtype=torch.int16, device="cuda")
    flat = flat_full[GUARD:]
    segs_dev = F.segments_to_device(segs)

    total = w.steps + w.warm_steps
    for t in range(1, total + 1):
        W.torch_grads_into(w, grads, t, seed)
        if pad_mask_dev is not None:
            for g in grads:
                g.masked_fill_(pad_mask_dev, 0x7FC0)
        kw = dict(step=t, segs=segs_dev, n_segments=L.n_segments, flat=flat,
                  flat_index0=lo - phase, lo=lo, **w.hp)
        if blocked:
            F.adamw_shard_step_blocked(state, grads, n=n, **kw)
        else:
            F.adamw_shard_step(master, m, v, grads, **kw)
        contribs = [g[idx_t].cpu().numpy().view(np.uint16) for g in grads]
        torch.cuda.synchronize()
        om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, w.hp, t)
        for k, want, what in ((0, om, "master"), (1, omm, "m"), (2, ov, "v")):
            _check(read[k](), want, f"{name} {what} step {t}")
        got = flat[phase:][idx_t].cpu().numpy().view(np.uint16)
        _check(got, oout, f"{name} bf16 step {t}")
        say(f"  step {t} ok")
    host_flat = flat_full.cpu().numpy().view(np.uint16)
    assert np.all(host_flat[:GUARD + phase] == SENT16), "flat prefix written"
    assert np.all(host_flat[GUARD + phase + n:] == SENT16), "flat suffix written"
    del grads, flat_full, read
    if blocked:
        del state, pos
    else:
        del master, m, v
    torch.cuda.empty_cache()


WORKLOAD_NAMES = ["p1000003_n8_rank3", "llama_layer_n8_rank0", "many_small_n16_rank3",
                  "dense7b_n8_rank0", "dense70b_n64_rank0"]


@pytest.mark.parametrize("blocked", [False, True], ids=["separate", "blocked"])
@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_fullsize(name, blocked):
    run_fullsize(name, blocked)


def _host_sumsq(g32, real_dev, chunk=1 << 26):
    """float64 sum of squares of the real elements of a device fp32 shard, computed on the host
    (chunk by chunk, each chunk's squares added by NumPy, the chunk sums added exactly)."""
    parts = []
    n = g32.numel()
    for a in range(0, n, chunk):
        x = g32[a:a + chunk][real_dev[a:a + chunk]].cpu().numpy().astype(np.float64)
        parts.append(float(np.dot(x, x)))
    return math.fsum(parts)


@pytest.mark.parametrize("name", ["dense7b_n8_rank0", "dense70b_n64_rank0"])
def test_clipped_fp32_path_full_size(name):
    """Clipping through an fp32 shard at full size, as the benchmark's clipped32 path runs it:
    reduce_shard_sumsq, then the clipped fp32-gradient step on the blocked state.  The fp32 shard
    is compared bit for bit with the oracle's reduction on the sampled windows; the fused float64
    sum, grad_sumsq_shard's sum over the same shard and grad_sumsq_shard's sum from the bf16
    contributions (too long for the oracle's exact sum) with a float64 sum of that shard taken on
    the host; the step on the windows with the oracle, whose
    clipping coefficient comes from the host's sum."""
    w = W.WORKLOADS[name]
    L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    lo_o, hi_o, osegs = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    n, lo = L.n, L.lo
    say(f"clipped fp32 path full size {name}: n={n} F={w.fan_in}")
    idx = _windows(n, [s["shard_begin"] for s in osegs[1:]], np.random.default_rng(5))
    idx_t = torch.from_numpy(idx).cuda()
    flags = _flags_at(osegs, idx)
    real_dev = torch.ones(n, dtype=torch.bool, device="cuda")
    for s in osegs:
        if s["flags"] & OL.PADDING:
            real_dev[s["shard_begin"]: s["shard_begin"] + s["length"]] = False
    segs_dev = F.segments_to_device(segs)

    master, m, v = W.torch_state(w, n, 2, "cuda")
    om, omm, ov = (x[idx_t].cpu().numpy() for x in (master, m, v))
    state = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device="cuda")
    F.state_to_blocked(master, m, v, state)
    del master, m, v
    grads = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(w.fan_in)]
    W.torch_grads_into(w, grads, 1, 2)
    g32 = torch.empty(n, dtype=torch.float32, device="cuda")
    sq = torch.zeros(1, dtype=torch.float64, device="cuda")
    scale = 0.5
    F.reduce_shard_sumsq(grads, g32, sq, scale=scale, segs=segs_dev, n_segments=L.n_segments)
    sq_bf16 = torch.zeros(1, dtype=torch.float64, device="cuda")     # from the contributions
    F.grad_sumsq_shard(sq_bf16, contribs=grads, n=n, scale=scale, segs=segs_dev,
                       n_segments=L.n_segments)
    contribs = [g[idx_t].cpu().numpy().view(np.uint16) for g in grads]
    del grads
    torch.cuda.synchronize()
    want32 = OS.reduce_contributions(contribs, scale)
    real = (flags & OL.PADDING) == 0
    got32 = g32[idx_t].cpu().numpy()
    assert np.array_equal(got32[real].view(np.uint32), want32[real].view(np.uint32))
    fused = float(sq.item())
    host = _host_sumsq(g32, real_dev)
    assert abs(fused - host) <= 1e-12 * host, (fused, host)
    sq2 = torch.zeros(1, dtype=torch.float64, device="cuda")
    F.grad_sumsq_shard(sq2, grad=g32, n=n, segs=segs_dev, n_segments=L.n_segments)
    assert abs(float(sq2.item()) - host) <= 1e-12 * host
    assert abs(float(sq_bf16.item()) - host) <= 1e-12 * host
    say(f"  fp32 shard and sums ok (sum {fused:.6e}, host {host:.6e})")

    max_norm = 0.5 * math.sqrt(host)                    # clipping on: coefficient about 1/2
    phase = lo % 8
    flat = torch.empty(phase + n, dtype=torch.int16, device="cuda")
    F.adamw_shard_step_f32grad_blocked(state, g32, step=1, n=n, segs=segs_dev,
                                       n_segments=L.n_segments, flat=flat,
                                       flat_index0=lo - phase, lo=lo, max_grad_norm=max_norm,
                                       grad_sumsq=sq, **w.hp)
    torch.cuda.synchronize()
    # The reference coefficient comes from the host's sum; the device used its own sum, which
    # differs in rounding order only, so bit equality is expected when both give one scale.
    coef_scale = OC.clipped_scale(host, max_norm)
    assert 0.4 < coef_scale < 0.6
    exact = OC.clipped_scale(fused, max_norm) == coef_scale
    om, omm, ov, oout = OS.shard_step_f32grad(om, omm, ov, want32, flags,
                                              dict(w.hp, grad_scale=float(coef_scale)), 1)
    for k, want, what in ((0, om, "master"), (1, omm, "m"), (2, ov, "v")):
        got = state[torch.from_numpy(_blocked_index(idx, k)).cuda()].cpu().numpy()
        _check(got, want, f"{name} clipped fp32 {what}", exact)
    got = flat[phase:][idx_t].cpu().numpy().view(np.uint16)
    _check(got, oout, f"{name} clipped fp32 bf16", exact)
    del state, g32, flat
    torch.cuda.empty_cache()


def test_slice_beyond_2_31_elements():
    """A slice longer than 2^31 elements (one tensor of 2^31 + 777, fan-in 1, blocked state), so
    every 32-bit boundary of element, vector and partial indices is crossed: two steps compared
    bit for bit with the oracle on windows at the start, across 2^31 and at the end; the sum of
    squares (65,537 partials) against a float64 sum of the inputs taken on the host; the
    allocation-free sum of squares refuses the length (its array holds 65,536 partials)."""
    n = (1 << 31) + 777
    w = W.Workload("beyond_2_31", "one tensor of 2^31 + 777 elements", [n], 1, 1, 0, 1, 2,
                   1e-3, ("normal", 0.02))
    L, segs = F.shard_layout(w.sizes, 1, 0)
    lo_o, hi_o, osegs = OL.segments(w.sizes, 1, None, 1, 0)
    assert (L.lo, L.n, L.n_segments) == (0, n, 1) and (lo_o, hi_o) == (0, n)
    say(f"slice beyond 2^31: n={n}")
    rng = np.random.default_rng(31)
    spans = [(0, WIN), ((1 << 31) - WIN, (1 << 31) + WIN), (n - WIN, n)]
    spans += [(int(s), int(s) + WIN) for s in rng.integers(0, n - WIN, 16)]
    idx = np.unique(np.concatenate([np.arange(a, min(b, n), dtype=np.int64) for a, b in spans]))
    idx_t = torch.from_numpy(idx).cuda()
    flags = _flags_at(osegs, idx)
    segs_dev = F.segments_to_device(segs)
    master, m, v = W.torch_state(w, n, 3, "cuda")
    om, omm, ov = (x[idx_t].cpu().numpy() for x in (master, m, v))
    state = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device="cuda")
    F.state_to_blocked(master, m, v, state)
    torch.cuda.synchronize()
    del master, m, v
    torch.cuda.empty_cache()
    pos = [torch.from_numpy(_blocked_index(idx, k)).cuda() for k in range(3)]
    grads = [torch.empty(n, dtype=torch.int16, device="cuda")]
    flat = torch.full((n,), int(SENT16), dtype=torch.int16, device="cuda")
    for t in (1, 2):
        W.torch_grads_into(w, grads, t, 3)
        F.adamw_shard_step_blocked(state, grads, step=t, n=n, segs=segs_dev,
                                   n_segments=L.n_segments, flat=flat, flat_index0=0, lo=0,
                                   **w.hp)
        contribs = [grads[0][idx_t].cpu().numpy().view(np.uint16)]
        torch.cuda.synchronize()
        om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, w.hp, t)
        for k, want, what in ((0, om, "master"), (1, omm, "m"), (2, ov, "v")):
            _check(state[pos[k]].cpu().numpy(), want, f"beyond 2^31 {what} step {t}")
        _check(flat[idx_t].cpu().numpy().view(np.uint16), oout, f"beyond 2^31 bf16 step {t}")
        say(f"  step {t} ok")
    del state, pos, flat
    torch.cuda.empty_cache()

    sq = torch.zeros(1, dtype=torch.float64, device="cuda")
    assert F.grad_sumsq_workspace_bytes(n) == 8 * 65_537
    F.grad_sumsq_shard(sq, contribs=grads, n=n, segs=segs_dev, n_segments=L.n_segments)
    parts = []
    chunk = 1 << 27
    for a in range(0, n, chunk):
        bits = grads[0][a:a + chunk].cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        x = bits.view(np.float32).astype(np.float64)
        parts.append(float(np.dot(x, x)))
    host = math.fsum(parts)
    assert abs(float(sq.item()) - host) <= 1e-12 * host, (float(sq.item()), host)
    with pytest.raises(F.FsdpShardError) as e:
        F.grad_sumsq_shard_noalloc(sq, contribs=grads, n=n)
    assert e.value.code == 3
    del grads
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fan_in", [2, 3, 16])
def test_large_slice_other_fan_ins(fan_in):
    """Fan-ins 2, 3 (the run-time loop) and 16 on a ragged slice of 2^27 + 123 elements, long
    enough for their 2-work-groups-per-CU launch, blocked and separate state alike: two steps
    compared bit for bit with the oracle on sampled windows (start, end, random)."""
    n = (1 << 27) + 123
    w = W.Workload(f"large_f{fan_in}", "one tensor of 2^27 + 123 elements", [n], 1, 1, 0,
                   fan_in, 2, 1e-3, ("uniform", 0.05))
    L, segs = F.shard_layout(w.sizes, 1, 0)
    _, _, osegs = OL.segments(w.sizes, 1, None, 1, 0)
    say(f"large slice, fan-in {fan_in}: n={n}")
    rng = np.random.default_rng(fan_in)
    idx = _windows(n, [], rng)
    idx_t = torch.from_numpy(idx).cuda()
    flags = _flags_at(osegs, idx)
    segs_dev = F.segments_to_device(segs)
    grads = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(fan_in)]
    for blocked in (True, False):
        master, m, v = W.torch_state(w, n, 11, "cuda")
        om, omm, ov = (x[idx_t].cpu().numpy() for x in (master, m, v))
        if blocked:
            state = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device="cuda")
            F.state_to_blocked(master, m, v, state)
            torch.cuda.synchronize()
            del master, m, v
            pos = [torch.from_numpy(_blocked_index(idx, k)).cuda() for k in range(3)]
            read = [lambda k=k: state[pos[k]].cpu().numpy() for k in range(3)]
        else:
            read = [lambda x=x: x[idx_t].cpu().numpy() for x in (master, m, v)]
        flat = torch.full((n,), int(SENT16), dtype=torch.int16, device="cuda")
        for t in (1, 2):
            W.torch_grads_into(w, grads, t, 11)
            kw = dict(step=t, segs=segs_dev, n_segments=L.n_segments, flat=flat, flat_index0=0,
                      lo=0, **w.hp)
            if blocked:
                F.adamw_shard_step_blocked(state, grads, n=n, **kw)
            else:
                F.adamw_shard_step(master, m, v, grads, **kw)
            contribs = [g[idx_t].cpu().numpy().view(np.uint16) for g in grads]
            torch.cuda.synchronize()
            om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, w.hp, t)
            what = f"fan-in {fan_in} {'blocked' if blocked else 'separate'}"
            for k, want, name in ((0, om, "master"), (1, omm, "m"), (2, ov, "v")):
                _check(read[k](), want, f"{what} {name} step {t}")
            _check(flat[idx_t].cpu().numpy().view(np.uint16), oout, f"{what} bf16 step {t}")
        say(f"  {'blocked' if blocked else 'separate'} ok")
        del read, flat
        if blocked:
            del state, pos
        else:
            del master, m, v
        torch.cuda.empty_cache()
    del grads
    torch.cuda.empty_cache()
