"""GPU parity of fp32 gradient accumulation, the fp32-gradient step, the sharded gradient norm
and clipping, against the oracle.

Bars: fp32 state relative 1e-5, bf16 within 1 ulp (as the step's other tests); the float64 sum of
squares relative 1e-12 against the oracle's exactly rounded sum (the kernel adds in a fixed tree
order, at most ~log2(n) + n/(32768*256) roundings of 2^-53 each), and bit-identical on repeat.
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
from gpu_helpers import Guarded, assert_bf16, assert_f32, bit_equal, say, to_dev16

pytestmark = pytest.mark.gpu
HP = dict(W.ADAMW)
SUMSQ_RTOL = 1e-12


def _layout(sizes, pad, wd, N, k):
    L, segs = F.shard_layout(sizes, N, k, pad, wd)
    lo, hi, osegs = OL.segments(sizes, pad, wd, N, k)
    flags = np.zeros(hi - lo, dtype=np.int64)
    for s in osegs:
        flags[s["shard_begin"]: s["shard_begin"] + s["length"]] = s["flags"]
    return L, segs, flags


@pytest.mark.parametrize("n,F_in,mbs", [(1, 1, 2), (4103, 3, 4), (65539, 8, 3), (300001, 2, 2)])
def test_accumulate_microbatches(n, F_in, mbs):
    say(f"accumulate n={n} F={F_in} micro-batches={mbs}")
    acc0 = W.np_f32_normal([60, n], n, 1e-3)
    acc = Guarded(acc0)
    want = acc0.copy()
    for mb in range(mbs):
        contribs = [W.np_bf16_normal([61, mb, r], n, 1e-2) for r in range(F_in)]
        F.reduce_shard_accumulate([to_dev16(c) for c in contribs], acc.data(), scale=0.25)
        want = OS.accumulate_fp32(want, contribs, 0.25)
    torch.cuda.synchronize()
    assert_f32(acc.data_host(), want, "accumulated gradient")
    assert bit_equal(acc.data_host(), want)
    acc.assert_guards("acc")


@pytest.mark.parametrize("d", [0, 3, 7])
@pytest.mark.parametrize("case", [None, ([5000, 3, 12000, 1, 1, 1, 7777], 8, [1, 0, 1, 1, 0, 1, 0], 3, 1)])
def test_f32grad_step(d, case):
    if case is None:
        n, lo, segs_dev, nseg = 100_003, 4000, None, 0
        flags = np.full(n, OL.WEIGHT_DECAY)
    else:
        L, segs, flags = _layout(*case)
        n, lo, nseg = L.n, L.lo, L.n_segments
        segs_dev = F.segments_to_device(segs)
    say(f"f32grad step n={n} d={d} segs={nseg}")
    master = W.np_f32_normal([62, 1], n, 0.02)
    m0 = W.np_f32_normal([62, 2], n, 1e-3)
    v0 = (W.np_f32_normal([62, 3], n, 1e-3) ** 2).astype(np.float32)
    gm, gmm, gv = Guarded(master), Guarded(m0), Guarded(v0)
    flat = Guarded(np.zeros(n, np.uint16), pre=d)
    om, omm, ov = master, m0, v0
    hp = dict(HP, grad_scale=0.5)
    for t in (1, 2):
        grad = W.np_f32_normal([63, t], n, 1e-2)
        grad[(flags & OL.PADDING) != 0] = np.nan
        gg = Guarded(grad)
        F.adamw_shard_step_f32grad(gm.data(), gmm.data(), gv.data(), gg.data(), step=t,
                                   segs=segs_dev, n_segments=nseg, flat=flat.window(),
                                   flat_index0=lo - d, lo=lo, **hp)
        torch.cuda.synchronize()
        om, omm, ov, oout = OS.shard_step_f32grad(om, omm, ov, grad, flags, hp, t)
        assert_f32(gm.data_host(), om, f"master step {t}")
        assert_f32(gmm.data_host(), omm, f"m step {t}")
        assert_f32(gv.data_host(), ov, f"v step {t}")
        assert_bf16(flat.data_host(), oout, f"bf16 step {t}")
        assert bit_equal(gm.data_host(), om) and bit_equal(flat.data_host(), oout)
        gg.assert_guards("grad")
    for g, what in ((gm, "master"), (gmm, "m"), (gv, "v"), (flat, "flat")):
        g.assert_guards(what)


def _gpu_sumsq(contribs=None, grad=None, n=None, scale=1.0, segs=None, nseg=0):
    out = torch.full((2,), float("nan"), dtype=torch.float64, device="cuda")
    F.grad_sumsq_shard(out[:1], contribs=contribs, grad=grad, n=n, scale=scale, segs=segs,
                       n_segments=nseg)
    torch.cuda.synchronize()
    h = out.cpu().numpy()
    assert np.isnan(h[1])                      # nothing written past the result
    return float(h[0])


@pytest.mark.parametrize("n,F_in", [(0, 2), (1, 1), (7, 8), (513, 3), (32768, 4), (32769, 8),
                                    (1_000_003, 8), (2_500_001, 1), (300_017, 5)])
def test_sumsq_matches_exact_sum(n, F_in):
    say(f"sumsq n={n} F={F_in}")
    contribs = [W.np_bf16_normal([64, r], n, 1e-2) for r in range(F_in)]
    dev = [to_dev16(c) if n else torch.zeros(8, dtype=torch.int16, device="cuda") for c in contribs]
    got = _gpu_sumsq(contribs=dev, n=n, scale=0.5)
    want = OC.grad_sumsq(contribs, np.ones(n, bool), 0.5) if n else 0.0
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)
    assert _gpu_sumsq(contribs=dev, n=n, scale=0.5) == got        # fixed order: bit-identical


def test_sumsq_fp32_grad_and_padding():
    L, segs, flags = _layout([5000, 3, 12000, 1, 1, 1, 77777], 16, None, 3, 1)
    n = L.n
    real = (flags & OL.PADDING) == 0
    grad = W.np_f32_normal([65, 1], n, 1e-2)
    grad[~real] = np.nan                                          # padding must not count
    gdev = torch.from_numpy(grad).cuda()
    got = _gpu_sumsq(grad=gdev, n=n, scale=2.0, segs=F.segments_to_device(segs), nseg=L.n_segments)
    want = OC.sumsq_exact(grad * np.float32(2.0), real)
    assert abs(got - want) <= SUMSQ_RTOL * want
    contribs = [W.np_bf16_normal([66, r], n, 1e-2) for r in range(4)]
    for c in contribs:
        c[~real] = 0x7FC0
    got = _gpu_sumsq(contribs=[to_dev16(c) for c in contribs], n=n,
                     segs=F.segments_to_device(segs), nseg=L.n_segments)
    want = OC.grad_sumsq(contribs, real)
    assert abs(got - want) <= SUMSQ_RTOL * want


@pytest.mark.parametrize("n", [32768, 32769, 262144 + 8, 1_000_003, 2_500_001])
def test_sumsq_fp32_grad_sizes(n):
    # Several whole 32,768-element tiles (the straight-line path, 8 groups per batch) and a tail.
    say(f"sumsq fp32 n={n}")
    grad = W.np_f32_normal([67, n], n, 1e-2)
    got = _gpu_sumsq(grad=torch.from_numpy(grad).cuda(), n=n, scale=0.25)
    want = OC.sumsq_exact(grad * np.float32(0.25))
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)


@pytest.mark.parametrize("blocks,tail", [(3840, 0), (3841, 1), (5000, 12345), (8192, 32767)])
def test_sumsq_finish_over_many_partials(blocks, tail):
    """Thousands of float64 partials, so the finish kernel's batched loads and its tail loop both
    run.  Element i holds 2^-4 * (1 + (i // 32768) % 3): every square is a power-of-two multiple
    of 2^-8, so the float64 sum is exact in any order and must equal sum(k^2) * 2^-8 bit for bit;
    a partial dropped or added twice changes it."""
    tile = 32768                               # elements per float64 partial
    n = blocks * tile + tail
    say(f"sumsq finish: n={n} partials={blocks + (tail > 0)}")
    idx = torch.arange(n, device="cuda", dtype=torch.int64)
    grad = ((idx // tile) % 3 + 1).to(torch.float32) * 0.0625
    del idx
    got = _gpu_sumsq(grad=grad, n=n)
    k = np.arange(blocks + 1, dtype=np.int64) % 3 + 1
    units = int((k[:blocks] ** 2).sum()) * tile + int(k[blocks] ** 2) * tail
    want = math.ldexp(units, -8)
    assert got == want, (got, want)
    del grad
    torch.cuda.empty_cache()


@pytest.mark.parametrize("F_in", [-1, 1, 4, 8])
def test_sumsq_padding_inside_whole_tiles(F_in):
    # 300 small tensors padded to 16 (padding every few hundred elements, NaN-filled) across
    # many whole tiles: the straight-line path must drop padding exactly as the checked path.
    sizes = [(i * 7919) % 3001 + 1 for i in range(300)]
    L, segs, flags = _layout(sizes, 16, None, 2, 1)
    n = L.n
    real = (flags & OL.PADDING) == 0
    say(f"sumsq padded tiles F={F_in} n={n} segments={L.n_segments}")
    sd, ns = F.segments_to_device(segs), L.n_segments
    if F_in == -1:
        grad = W.np_f32_normal([68, 1], n, 1e-2)
        grad[~real] = np.nan
        got = _gpu_sumsq(grad=torch.from_numpy(grad).cuda(), n=n, segs=sd, nseg=ns)
        want = OC.sumsq_exact(grad, real)
    else:
        contribs = [W.np_bf16_normal([69, r], n, 1e-2) for r in range(F_in)]
        for c in contribs:
            c[~real] = 0x7FC0
        got = _gpu_sumsq(contribs=[to_dev16(c) for c in contribs], n=n, segs=sd, nseg=ns)
        want = OC.grad_sumsq(contribs, real)
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)


@pytest.mark.parametrize("max_norm", [1e-3, 0.5, 1e9])
def test_clipped_step_all_ranks(max_norm):
    """Every rank of a small model computes its part of the squared norm on the GPU; the parts
    are added in rank order (the one-GPU stand-in for the scalar all-reduce) and every rank clips
    with the global norm.  The union of the ranks' results equals the oracle's clipped step of
    the whole flat vector, where the oracle computes the norm itself."""
    sizes, pad, wd, N, Fi = [3000, 17, 1, 40000, 5, 26000, 999], 16, [1, 0, 1, 1, 0, 1, 0], 4, 3
    offs, P = OL.flatten_offsets(sizes, pad)
    flags_full = np.zeros(P, dtype=np.int64)
    ranks = []
    for k in range(N):
        L, segs, fl = _layout(sizes, pad, wd, N, k)
        flags_full[L.lo:L.hi] = fl
        ranks.append((L, F.segments_to_device(segs)))
    real_full = (flags_full & OL.PADDING) == 0
    master = W.np_f32_normal([67, 1], P, 0.02)
    flat = Guarded(np.zeros(P, np.uint16))
    state = []
    for L, _ in ranks:
        state.append([Guarded(master[L.lo:L.hi]), Guarded(np.zeros(L.n, np.float32)),
                      Guarded(np.zeros(L.n, np.float32))])
    om, omm, ov = master, np.zeros(P, np.float32), np.zeros(P, np.float32)
    for t in (1, 2):
        grads = [W.np_bf16_normal([68, t, r], P, 1e-2) for r in range(Fi)]
        for g in grads:
            g[~real_full] = 0x7FC0
        parts, devs = [], []
        for (L, sd) in ranks:
            dev = [to_dev16(g[L.lo:L.hi]) for g in grads]
            devs.append(dev)
            parts.append(_gpu_sumsq(contribs=dev, n=L.n, segs=sd, nseg=L.n_segments))
        total = 0.0
        for x in parts:                       # rank order
            total += x
        tdev = torch.tensor([total], dtype=torch.float64, device="cuda")
        for (L, sd), st, dev in zip(ranks, state, devs):
            F.adamw_shard_step(st[0].data(), st[1].data(), st[2].data(), dev, step=t, segs=sd,
                               n_segments=L.n_segments, flat=flat.window(), flat_index0=0,
                               lo=L.lo, max_grad_norm=max_norm, grad_sumsq=tdev, **HP)
        torch.cuda.synchronize()
        osum = OC.grad_sumsq(grads, real_full)
        assert abs(total - osum) <= SUMSQ_RTOL * osum
        assert max(parts) < osum                  # each rank alone underestimates the norm
        scale = OC.clipped_scale(osum, max_norm)
        om, omm, ov, oout = OS.shard_step(om, omm, ov, grads, flags_full,
                                          dict(HP, grad_scale=float(scale)), t)
        assert_bf16(flat.data_host(), oout, f"flat step {t}")
        for (L, _), st in zip(ranks, state):
            assert_f32(st[0].data_host(), om[L.lo:L.hi], "master")
            assert_f32(st[1].data_host(), omm[L.lo:L.hi], "m")
            assert_f32(st[2].data_host(), ov[L.lo:L.hi], "v")
    flat.assert_guards("flat")
    if max_norm >= 1e9:
        assert OC.clip_coefficient(osum, max_norm) == 1.0


def test_clipped_f32grad_step_matches_oracle():
    n = 70_001
    master = W.np_f32_normal([69, 1], n, 0.02)
    grad = W.np_f32_normal([69, 2], n, 1.0)
    gm = Guarded(master)
    gmm, gv = Guarded(np.zeros(n, np.float32)), Guarded(np.zeros(n, np.float32))
    flat = Guarded(np.zeros(n, np.uint16), pre=5)
    gdev = torch.from_numpy(grad).cuda()
    sq = torch.zeros(1, dtype=torch.float64, device="cuda")
    F.grad_sumsq_shard(sq, grad=gdev, n=n)
    F.adamw_shard_step_f32grad(gm.data(), gmm.data(), gv.data(), gdev, step=1,
                               flat=flat.window(), flat_index0=995, lo=1000, max_grad_norm=1.0,
                               grad_sumsq=sq, **HP)
    torch.cuda.synchronize()
    osum = OC.sumsq_exact(grad)
    scale = OC.clipped_scale(osum, 1.0)
    assert scale < 0.01                                            # the norm is ~sqrt(n)
    flags = np.full(n, OL.WEIGHT_DECAY)
    om, omm, ov, oout = OS.shard_step_f32grad(master, np.zeros(n, np.float32),
                                              np.zeros(n, np.float32), grad, flags,
                                              dict(HP, grad_scale=float(scale)), 1)
    assert_f32(gm.data_host(), om, "master")
    assert_f32(gmm.data_host(), omm, "m")
    assert_bf16(flat.data_host(), oout, "bf16")
    assert bit_equal(gmm.data_host(), omm)


@pytest.mark.slow
def test_sumsq_llama_layer_full_slice():
    """Full 27,264,000-element slice of one Llama-style layer, fan-in 8, against the exact sum."""
    w = W.WORKLOADS["llama_layer_n8_rank0"]
    L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    grads = [torch.empty(L.n, dtype=torch.int16, device="cuda") for _ in range(w.fan_in)]
    W.torch_grads_into(w, grads, 1, 3)
    got = _gpu_sumsq(contribs=grads, n=L.n, segs=F.segments_to_device(segs), nseg=L.n_segments)
    host = [g.cpu().numpy().view(np.uint16) for g in grads]
    want = OC.grad_sumsq(host, np.ones(L.n, bool))
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dense7b_n8_rank0", "dense70b_n64_rank0"])
def test_sumsq_full_slice_parts_add_up(name):
    """At 7B / 70B size: the slice's sum equals the sum of four sub-slices' sums (a property at
    any size) and the first 4 Mi elements match the oracle's exact sum."""
    w = W.WORKLOADS[name]
    L, _ = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    n = L.n
    grads = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(w.fan_in)]
    W.torch_grads_into(w, grads, 1, 4)
    whole = _gpu_sumsq(contribs=grads, n=n)
    cuts = [0, n // 4 // 8 * 8, n // 2 // 8 * 8, 3 * n // 4 // 8 * 8, n]
    parts = [_gpu_sumsq(contribs=[g[a:b] for g in grads], n=b - a) for a, b in zip(cuts, cuts[1:])]
    assert abs(sum(parts) - whole) <= SUMSQ_RTOL * whole
    k = 1 << 22
    head = _gpu_sumsq(contribs=[g[:k] for g in grads], n=k)
    want = OC.grad_sumsq([g[:k].cpu().numpy().view(np.uint16) for g in grads], np.ones(k, bool))
    assert abs(head - want) <= SUMSQ_RTOL * want
    assert math.isfinite(whole) and whole > 0
    del grads
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n,F_in,acc", [(1, 1, False), (7, 3, True), (32768, 8, False),
                                        (32769, 8, True), (65539, 2, True), (300_017, 5, False),
                                        (1_000_003, 1, True), (2_500_001, 4, False),
                                        (1_000_003, 4, True), (300_017, 8, True),
                                        (2_500_001, 8, False), (98_304, 4, True)])
def test_reduce_sumsq_matches_oracle(n, F_in, acc):
    # The fp32 shard equals the plain reduction (or accumulation) bit for bit; the sum of squares
    # of that shard matches the oracle's exact sum; the sum is bit-identical when repeated.
    say(f"reduce+sumsq n={n} F={F_in} accumulate={acc}")
    contribs = [W.np_bf16_normal([70, r], n, 1e-2) for r in range(F_in)]
    dev = [to_dev16(c) for c in contribs]
    acc0 = W.np_f32_normal([71, n], n, 1e-3) if acc else np.full(n, np.nan, np.float32)
    out = Guarded(acc0)
    res = torch.full((2,), float("nan"), dtype=torch.float64, device="cuda")
    F.reduce_shard_sumsq(dev, out.data(), res[:1], accumulate=acc, scale=0.5)
    torch.cuda.synchronize()
    want = OS.accumulate_fp32(acc0, contribs, 0.5) if acc else OS.reduce_contributions(contribs, 0.5)
    assert bit_equal(out.data_host(), want)
    out.assert_guards("out")
    h = res.cpu().numpy()
    assert np.isnan(h[1])
    osum = OC.sumsq_exact(want)
    assert abs(h[0] - osum) <= SUMSQ_RTOL * osum, (h[0], osum)
    if not acc:
        F.reduce_shard_sumsq(dev, out.data(), res[:1], scale=0.5)
        torch.cuda.synchronize()
        assert res.cpu().numpy()[0] == h[0]
        # The fused sum agrees with grad_sumsq_shard over the same fp32 shard.
        assert abs(_gpu_sumsq(grad=out.data(), n=n) - h[0]) <= SUMSQ_RTOL * osum


@pytest.mark.parametrize("F_in,acc", [(8, False), (8, True), (4, True), (4, False), (1, False),
                                      (2, True)])
def test_reduce_sumsq_padding_inside_whole_tiles(F_in, acc):
    # A padded layout across several whole tiles (the straight-line paths, pipelined or not):
    # the fp32 shard is the plain reduction bit for bit and the sum drops every padding element.
    sizes = [(i * 7919) % 3001 + 1 for i in range(300)]
    L, segs, flags = _layout(sizes, 16, None, 2, 1)
    n = L.n
    real = (flags & OL.PADDING) == 0
    say(f"reduce+sumsq padded tiles F={F_in} accumulate={acc} n={n} segments={L.n_segments}")
    contribs = [W.np_bf16_normal([74, r], n, 1e-2) for r in range(F_in)]
    for c in contribs:
        c[~real] = 0x7FC0
    acc0 = W.np_f32_normal([75, n], n, 1e-3) if acc else np.zeros(n, np.float32)
    out = Guarded(acc0)
    res = torch.zeros(1, dtype=torch.float64, device="cuda")
    F.reduce_shard_sumsq([to_dev16(c) for c in contribs], out.data(), res, accumulate=acc,
                         scale=0.25, segs=F.segments_to_device(segs), n_segments=L.n_segments)
    torch.cuda.synchronize()
    want = (OS.accumulate_fp32(acc0, contribs, 0.25) if acc
            else OS.reduce_contributions(contribs, 0.25))
    assert n > 4 * 32768
    assert bit_equal(out.data_host()[real], want[real])
    out.assert_guards("out")
    osum = OC.sumsq_exact(want, real)
    got = float(res.cpu().numpy()[0])
    assert abs(got - osum) <= SUMSQ_RTOL * osum, (got, osum)


@pytest.mark.parametrize("F_in", [1, 4, 8, 3])
def test_microbatches_with_fused_norm_then_clipped_step(F_in):
    # Three micro-batches: reduce, accumulate, then accumulate fused with the sum of squares; the
    # clipped fp32-gradient step uses that norm.  Padding (NaN contributions) never counts.
    sizes = [(i * 7919) % 3001 + 1 for i in range(300)]
    L, segs, flags = _layout(sizes, 16, [i % 3 != 0 for i in range(300)], 2, 1)
    n = L.n
    real = (flags & OL.PADDING) == 0
    sd = F.segments_to_device(segs)
    say(f"micro-batches + fused norm F={F_in} n={n} segments={L.n_segments}")
    mbs = []
    for mb in range(3):
        cs = [W.np_bf16_normal([72, mb, r], n, 1e-2) for r in range(F_in)]
        for c in cs:
            c[~real] = 0x7FC0
        mbs.append(cs)
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    res = torch.zeros(1, dtype=torch.float64, device="cuda")
    F.reduce_shard([to_dev16(c) for c in mbs[0]], acc)
    F.reduce_shard_accumulate([to_dev16(c) for c in mbs[1]], acc)
    F.reduce_shard_sumsq([to_dev16(c) for c in mbs[2]], acc, res, accumulate=True, segs=sd,
                         n_segments=L.n_segments)
    oacc = OS.reduce_contributions(mbs[0])
    oacc = OS.accumulate_fp32(oacc, mbs[1])
    oacc = OS.accumulate_fp32(oacc, mbs[2])
    torch.cuda.synchronize()
    got_acc = acc.cpu().numpy()
    assert bit_equal(got_acc[real], oacc[real])
    osum = OC.sumsq_exact(oacc, real)
    total = float(res.cpu().numpy()[0])
    assert abs(total - osum) <= SUMSQ_RTOL * osum
    master = W.np_f32_normal([73, 1], n, 0.02)
    st = [Guarded(master), Guarded(np.zeros(n, np.float32)), Guarded(np.zeros(n, np.float32))]
    flat = Guarded(np.zeros(n, np.uint16))
    max_norm = 0.05
    F.adamw_shard_step_f32grad(st[0].data(), st[1].data(), st[2].data(), acc, step=1, segs=sd,
                               n_segments=L.n_segments, flat=flat.window(), flat_index0=L.lo,
                               lo=L.lo, max_grad_norm=max_norm, grad_sumsq=res, **HP)
    torch.cuda.synchronize()
    scale = OC.clipped_scale(osum, max_norm)
    assert scale < 1.0                                   # the clip is active in this case
    om, omm, ov, oout = OS.shard_step_f32grad(master, np.zeros(n, np.float32),
                                              np.zeros(n, np.float32), oacc, flags,
                                              dict(HP, grad_scale=float(scale)), 1)
    assert_f32(st[0].data_host(), om, "master")
    assert_f32(st[1].data_host(), omm, "m")
    assert_f32(st[2].data_host(), ov, "v")
    assert_bf16(flat.data_host(), oout, "flat")
    for g, what in zip(st + [flat], ("master", "m", "v", "flat")):
        g.assert_guards(what)
