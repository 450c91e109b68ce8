"""Randomized GPU parity sweep of the fused step against the oracle.

Each trial draws a whole case from a seeded generator: tensor sizes and padding multiple, world
size and rank, per-tensor weight-decay mask, fan-in (compile-time and run-time fan-ins up to 64)
or an fp32 gradient shard, AdamW hyperparameters, gradient scale, clipping by the global norm
(the squared norm taken on the GPU, as a caller would; with bf16 contributions either from the
contributions or from the fp32 shard that reduce_shard_sumsq writes) and the bf16 window's phase.
Two steps per trial; fp32 state within relative 1e-5, bf16 within 1 ulp, NaN padding gradients
ignored, guard bands intact.  The library is also expected to equal the oracle bit for bit (same
operations in the same order, no contraction, IEEE division and square root); with clipping that
holds whenever the float32 scale formed from the device's sum of squares equals the one formed
from the oracle's exactly rounded sum (the two sums differ in rounding order only).
"""

import random

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from oracle import clip as OC
from oracle import layout as OL
from oracle import step as OS
import blocked_layout as BL
from gpu_helpers import Guarded, assert_bf16, assert_f32, bit_equal, say, to_dev16

pytestmark = pytest.mark.gpu
SIZE_CHOICES = [1, 3, 7, 16, 100, 513, 2049, 4099, 30001, 70003]
FAN_CHOICES = [-1, 1, 2, 3, 4, 5, 7, 8, 9, 16, 33, 64]   # -1: one fp32 gradient shard


def _draw(rng):
    while True:
        T = rng.randint(1, 8)
        sizes = [rng.choice(SIZE_CHOICES) for _ in range(T)]
        pad = rng.choice([1, 2, 4, 8, 16])
        N = rng.randint(1, 9)
        k = rng.randrange(N)
        _, P = OL.flatten_offsets(sizes, pad)
        lo, hi = OL.shard_bounds(P, N, k)
        if hi > lo:
            break
    wd = [int(rng.random() < 0.6) for _ in range(T)]
    hp = dict(lr=rng.choice([1e-3, 3e-4, 1e-2]), beta1=rng.choice([0.9, 0.8]),
              beta2=rng.choice([0.999, 0.95]), eps=rng.choice([1e-8, 1e-6]),
              weight_decay=rng.choice([0.0, 0.01, 0.1]),
              grad_scale=rng.choice([1.0, 0.5, 0.125]))
    return dict(sizes=sizes, pad=pad, N=N, k=k, wd=wd, F_in=rng.choice(FAN_CHOICES), hp=hp,
                clip=rng.choice([0.0, 0.0, 1e-3, 10.0]), d=rng.randrange(32))


def _same_scale(sumsq, clip, base, oracle_scale):
    """Whether the float32 clip scale formed from the device's sum of squares equals the one the
    oracle formed from its exactly rounded sum (then the steps must agree bit for bit)."""
    torch.cuda.synchronize()
    return float(OC.clipped_scale(float(sumsq.item()), clip, base)) == oracle_scale


def _check_step(got, want, t, exact):
    """Tolerance checks of one step (fp32 relative 1e-5, bf16 1 ulp), then bit equality."""
    for (g, w), what in zip(zip(got, want), ("master", "m", "v")):
        assert_f32(g, w, f"{what} step {t}")
    assert_bf16(got[3], want[3], f"bf16 step {t}")
    if exact:
        for (g, w), what in zip(zip(got, want), ("master", "m", "v", "bf16")):
            assert bit_equal(g, w), f"{what} step {t} not bit-equal to the oracle"


@pytest.mark.parametrize("trial", range(40))
def test_random_fused_steps(trial):
    c = _draw(random.Random(1000 + trial))
    L, segs = F.shard_layout(c["sizes"], c["N"], c["k"], c["pad"], c["wd"])
    lo, hi, osegs = OL.segments(c["sizes"], c["pad"], c["wd"], c["N"], c["k"])
    assert (L.lo, L.hi) == (lo, hi)
    n = hi - lo
    flags = np.zeros(n, dtype=np.int64)
    for s in osegs:
        flags[s["shard_begin"]: s["shard_begin"] + s["length"]] = s["flags"]
    real = (flags & OL.PADDING) == 0
    F_in, hp, clip, d = c["F_in"], c["hp"], c["clip"], c["d"]
    say(f"random trial {trial}: n={n} lo={lo} segs={L.n_segments} F={F_in} clip={clip} d={d} "
        f"hp={hp}")
    sd = F.segments_to_device(segs)
    seed = 5000 + trial
    master0 = W.np_f32_normal([seed, 1], n, 0.02)
    m0 = W.np_f32_normal([seed, 2], n, 1e-3)
    v0 = (np.abs(W.np_f32_normal([seed, 3], n, 1e-3)) ** 2).astype(np.float32)
    gm, gmm, gv = Guarded(master0), Guarded(m0), Guarded(v0)
    flat = Guarded(np.zeros(n, np.uint16), pre=d)
    om, omm, ov = master0.copy(), m0.copy(), v0.copy()
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in (1, 2):
        ohp = dict(hp)
        exact = True
        kw = dict(step=t, segs=sd, n_segments=L.n_segments, flat=flat.window(),
                  flat_index0=lo - d, lo=lo, **hp)
        if F_in == -1:
            grad = W.np_f32_normal([seed, 10 + t], n, 1e-2)
            grad[~real] = np.nan
            gdev = torch.from_numpy(grad).cuda()
            if clip:
                F.grad_sumsq_shard(sumsq, grad=gdev, n=n, scale=hp["grad_scale"], segs=sd,
                                   n_segments=L.n_segments)
                osum = OC.sumsq_exact(grad * np.float32(hp["grad_scale"]), real)
                ohp["grad_scale"] = float(OC.clipped_scale(osum, clip, hp["grad_scale"]))
                exact = _same_scale(sumsq, clip, hp["grad_scale"], ohp["grad_scale"])
                kw.update(max_grad_norm=clip, grad_sumsq=sumsq)
            F.adamw_shard_step_f32grad(gm.data(), gmm.data(), gv.data(), gdev, **kw)
            om, omm, ov, oout = OS.shard_step_f32grad(om, omm, ov, grad, flags, ohp, t)
        else:
            contribs = [W.np_bf16_normal([seed, 20 + t, r], n, 1e-2) for r in range(F_in)]
            for cb in contribs:
                cb[~real] = 0x7FC0
            dev = [to_dev16(cb) for cb in contribs]
            if clip and trial % 2:
                # Reduce once into an fp32 shard with its norm, then the fp32-gradient step.
                acc = torch.empty(n, dtype=torch.float32, device="cuda")
                F.reduce_shard_sumsq(dev, acc, sumsq, scale=hp["grad_scale"], segs=sd,
                                     n_segments=L.n_segments)
                ograd = OS.reduce_contributions(contribs, hp["grad_scale"])
                osum = OC.sumsq_exact(ograd, real)
                ohp["grad_scale"] = float(OC.clipped_scale(osum, clip, 1.0))
                exact = _same_scale(sumsq, clip, 1.0, ohp["grad_scale"])
                kw.update(max_grad_norm=clip, grad_sumsq=sumsq, grad_scale=1.0)
                F.adamw_shard_step_f32grad(gm.data(), gmm.data(), gv.data(), acc, **kw)
                om, omm, ov, oout = OS.shard_step_f32grad(om, omm, ov, ograd, flags, ohp, t)
                torch.cuda.synchronize()
                _check_step((gm.data_host(), gmm.data_host(), gv.data_host(), flat.data_host()),
                            (om, omm, ov, oout), t, exact)
                continue
            if clip:
                F.grad_sumsq_shard(sumsq, contribs=dev, n=n, scale=hp["grad_scale"],
                                   segs=sd, n_segments=L.n_segments)
                osum = OC.grad_sumsq(contribs, real, hp["grad_scale"])
                ohp["grad_scale"] = float(OC.clipped_scale(osum, clip, hp["grad_scale"]))
                exact = _same_scale(sumsq, clip, hp["grad_scale"], ohp["grad_scale"])
                kw.update(max_grad_norm=clip, grad_sumsq=sumsq)
            F.adamw_shard_step(gm.data(), gmm.data(), gv.data(), dev, **kw)
            om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, ohp, t)
        torch.cuda.synchronize()
        _check_step((gm.data_host(), gmm.data_host(), gv.data_host(), flat.data_host()),
                    (om, omm, ov, oout), t, exact)
    for g, what in ((gm, "master"), (gmm, "m"), (gv, "v"), (flat, "flat window")):
        g.assert_guards(what)


@pytest.mark.parametrize("trial", range(24))
def test_random_blocked_steps(trial):
    """The same randomized cases through the blocked-state entry points (the layout the
    benchmark times): bf16 contributions or an fp32 gradient shard, with or without clipping,
    against the oracle; slots past n in the last block and every guard band stay untouched."""
    c = _draw(random.Random(3000 + trial))
    L, segs = F.shard_layout(c["sizes"], c["N"], c["k"], c["pad"], c["wd"])
    lo, hi, osegs = OL.segments(c["sizes"], c["pad"], c["wd"], c["N"], c["k"])
    assert (L.lo, L.hi) == (lo, hi)
    n = hi - lo
    flags = np.zeros(n, dtype=np.int64)
    for s in osegs:
        flags[s["shard_begin"]: s["shard_begin"] + s["length"]] = s["flags"]
    real = (flags & OL.PADDING) == 0
    F_in, hp, clip, d = c["F_in"], c["hp"], c["clip"], c["d"]
    say(f"random blocked trial {trial}: n={n} lo={lo} segs={L.n_segments} F={F_in} clip={clip} "
        f"d={d} hp={hp}")
    sd = F.segments_to_device(segs)
    seed = 7000 + trial
    master0 = W.np_f32_normal([seed, 1], n, 0.02)
    m0 = W.np_f32_normal([seed, 2], n, 1e-3)
    v0 = (np.abs(W.np_f32_normal([seed, 3], n, 1e-3)) ** 2).astype(np.float32)
    unused = 0x7FB0B0B0
    blk = Guarded(BL.to_blocked(master0, m0, v0, fill=np.uint32(unused).view(np.float32)))
    flat = Guarded(np.zeros(n, np.uint16), pre=d)
    om, omm, ov = master0.copy(), m0.copy(), v0.copy()
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in (1, 2):
        ohp = dict(hp)
        exact = True
        kw = dict(step=t, segs=sd, n_segments=L.n_segments, flat=flat.window(),
                  flat_index0=lo - d, lo=lo, **hp)
        if F_in == -1:
            grad = W.np_f32_normal([seed, 10 + t], n, 1e-2)
            grad[~real] = np.nan
            gdev = torch.from_numpy(grad).cuda()
            if clip:
                F.grad_sumsq_shard(sumsq, grad=gdev, n=n, scale=hp["grad_scale"], segs=sd,
                                   n_segments=L.n_segments)
                osum = OC.sumsq_exact(grad * np.float32(hp["grad_scale"]), real)
                ohp["grad_scale"] = float(OC.clipped_scale(osum, clip, hp["grad_scale"]))
                exact = _same_scale(sumsq, clip, hp["grad_scale"], ohp["grad_scale"])
                kw.update(max_grad_norm=clip, grad_sumsq=sumsq)
            F.adamw_shard_step_f32grad_blocked(blk.data(), gdev, n=n, **kw)
            om, omm, ov, oout = OS.shard_step_f32grad(om, omm, ov, grad, flags, ohp, t)
        else:
            contribs = [W.np_bf16_normal([seed, 20 + t, r], n, 1e-2) for r in range(F_in)]
            for cb in contribs:
                cb[~real] = 0x7FC0
            dev = [to_dev16(cb) for cb in contribs]
            if clip:
                F.grad_sumsq_shard(sumsq, contribs=dev, n=n, scale=hp["grad_scale"], segs=sd,
                                   n_segments=L.n_segments)
                osum = OC.grad_sumsq(contribs, real, hp["grad_scale"])
                ohp["grad_scale"] = float(OC.clipped_scale(osum, clip, hp["grad_scale"]))
                exact = _same_scale(sumsq, clip, hp["grad_scale"], ohp["grad_scale"])
                kw.update(max_grad_norm=clip, grad_sumsq=sumsq)
            F.adamw_shard_step_blocked(blk.data(), dev, n=n, **kw)
            om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, ohp, t)
        torch.cuda.synchronize()
        gm, gmm, gv = BL.from_blocked(blk.data_host(), n)
        _check_step((gm, gmm, gv, flat.data_host()), (om, omm, ov, oout), t, exact)
    st = blk.data_host().view(np.uint32)
    used = BL.to_blocked(np.ones(n, np.float32), np.ones(n, np.float32), np.ones(n, np.float32),
                         fill=0.0) != 0.0
    assert (st[~used] == np.uint32(unused)).all(), "unused slots of the last block written"
    blk.assert_guards("blocked state")
    flat.assert_guards("flat window")
