"""Full-size parity: each shard configuration at its real shape, in the launch configuration the
benchmark times, compared with the oracle on sampled windows of the slice.

The step is elementwise once the layout is fixed, so the oracle can recompute any subset of
elements from the same inputs.  Windows: the first and last 1 Mi elements, +-4 Ki around every
segment edge inside the slice, and 64 random 64 Ki windows.  Inputs are drawn on the device with
seeded generators (no value comes from the library); the oracle receives copies of exactly the
windowed inputs.  The bf16 destination uses the phase the slice has in a 16-byte aligned flat
vector (lo mod 8), and a guarded prefix / suffix of the flat window must survive.
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
from gpu_helpers import SENT16, assert_bf16, assert_f32, say

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


def run_fullsize(name, seed=0, steps=None):
    w = W.WORKLOADS[name]
    L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    lo_o, hi_o, osegs = OL.segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    assert (L.lo, L.hi) == (lo_o, hi_o)
    n, lo = L.n, L.lo
    say(f"fullsize {name}: n={n} lo={lo} F={w.fan_in} segs={L.n_segments}")
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
    grads = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(w.fan_in)]
    phase = lo % 8
    GUARD = 64
    flat_full = torch.full((GUARD + phase + n + GUARD,), int(SENT16),
                           dtype=torch.int16, device="cuda")
    flat = flat_full[GUARD:]
    segs_dev = F.segments_to_device(segs)

    om = master[idx_t].cpu().numpy()
    omm = m[idx_t].cpu().numpy()
    ov = v[idx_t].cpu().numpy()
    total = (steps or w.steps) + w.warm_steps
    for t in range(1, total + 1):
        W.torch_grads_into(w, grads, t, seed)
        if pad_mask_dev is not None:
            for g in grads:
                g.masked_fill_(pad_mask_dev, 0x7FC0)
        F.adamw_shard_step(master, m, v, grads, step=t, segs=segs_dev, n_segments=L.n_segments,
                           flat=flat, flat_index0=lo - phase, lo=lo, **w.hp)
        contribs = [g[idx_t].cpu().numpy().view(np.uint16) for g in grads]
        torch.cuda.synchronize()
        om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, w.hp, t)
        assert_f32(master[idx_t].cpu().numpy(), om, f"{name} master step {t}")
        assert_f32(m[idx_t].cpu().numpy(), omm, f"{name} m step {t}")
        assert_f32(v[idx_t].cpu().numpy(), ov, f"{name} v step {t}")
        got = flat[phase:][idx_t].cpu().numpy().view(np.uint16)
        assert_bf16(got, oout, f"{name} bf16 step {t}")
        say(f"  step {t} ok")
    host_flat = flat_full.cpu().numpy().view(np.uint16)
    assert np.all(host_flat[:GUARD + phase] == SENT16), "flat prefix written"
    assert np.all(host_flat[GUARD + phase + n:] == SENT16), "flat suffix written"
    del master, m, v, grads, flat_full
    torch.cuda.empty_cache()


def test_p1000003_rank3():
    run_fullsize("p1000003_n8_rank3")


def test_llama_layer_with_warm_moments():
    run_fullsize("llama_layer_n8_rank0", steps=3)


def test_many_small_tensors():
    run_fullsize("many_small_n16_rank3")


def test_dense7b_slice():
    run_fullsize("dense7b_n8_rank0", steps=2)


def test_dense70b_slice():
    run_fullsize("dense70b_n64_rank0", steps=2)


def _blocked_index(idx, k):
    """Position of element idx's k-th state value (0 master, 1 m, 2 v) in the blocked array."""
    return ((idx // OL.STATE_BLOCK) * 3 + k) * OL.STATE_BLOCK + idx % OL.STATE_BLOCK


@pytest.mark.parametrize("name", ["dense7b_n8_rank0", "dense70b_n64_rank0"])
def test_clipped_fp32_path_full_size(name):
    """Clipping through an fp32 shard at full size, as the benchmark's clipped32 path runs it:
    reduce_shard_sumsq, then the clipped fp32-gradient step on the blocked state.  The fp32 shard
    is compared bit for bit with the oracle's reduction on the sampled windows; the fused float64
    sum (too long for the oracle's exact sum) with an independent float64 sum on the device and
    with grad_sumsq_shard over the same shard; the step on the windows with the oracle, whose
    clipping coefficient comes from that checked sum."""
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
    contribs = [g[idx_t].cpu().numpy().view(np.uint16) for g in grads]
    del grads
    torch.cuda.synchronize()
    want32 = OS.reduce_contributions(contribs, scale)
    real = (flags & OL.PADDING) == 0
    got32 = g32[idx_t].cpu().numpy()
    assert np.array_equal(got32[real].view(np.uint32), want32[real].view(np.uint32))
    fused = float(sq.item())
    indep = float((g32[real_dev].double() ** 2).sum().item())
    assert abs(fused - indep) <= 1e-12 * indep, (fused, indep)
    sq2 = torch.zeros(1, dtype=torch.float64, device="cuda")
    F.grad_sumsq_shard(sq2, grad=g32, n=n, segs=segs_dev, n_segments=L.n_segments)
    assert abs(float(sq2.item()) - fused) <= 1e-12 * fused
    say(f"  fp32 shard and sum ok (sum {fused:.6e})")

    max_norm = 0.5 * math.sqrt(fused)                   # clipping on: coefficient about 1/2
    phase = lo % 8
    flat = torch.empty(phase + n, dtype=torch.int16, device="cuda")
    F.adamw_shard_step_f32grad_blocked(state, g32, step=1, n=n, segs=segs_dev,
                                       n_segments=L.n_segments, flat=flat,
                                       flat_index0=lo - phase, lo=lo, max_grad_norm=max_norm,
                                       grad_sumsq=sq, **w.hp)
    torch.cuda.synchronize()
    coef_scale = OC.clipped_scale(fused, max_norm)
    assert 0.4 < coef_scale < 0.6
    om, omm, ov, oout = OS.shard_step_f32grad(om, omm, ov, want32, flags,
                                              dict(w.hp, grad_scale=float(coef_scale)), 1)
    for k, want, what in ((0, om, "master"), (1, omm, "m"), (2, ov, "v")):
        got = state[torch.from_numpy(_blocked_index(idx, k)).cuda()].cpu().numpy()
        assert_f32(got, want, f"{name} clipped fp32 {what}")
    got = flat[phase:][idx_t].cpu().numpy().view(np.uint16)
    assert_bf16(got, oout, f"{name} clipped fp32 bf16")
    del state, g32, flat
    torch.cuda.empty_cache()
