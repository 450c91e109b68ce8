"""GPU parity of the blocked state layout.

* state_to_blocked / state_from_blocked against the oracle's definition of the layout, bit for
  bit, with the unused slots of the last block and guard bands untouched;
* adamw_shard_step_blocked / adamw_shard_step_f32grad_blocked against the oracle (fp32 state
  within relative 1e-5, bf16 within 1 ulp) and bit for bit against the separate-layout calls on
  the same inputs, over sizes with ragged tails, fan-ins, segment tables with NaN padding
  gradients, all eight output phases and clipping;
* the 7B-shaped slice at full size: two blocked steps equal two separate-layout steps bit for bit.
"""

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
HP = dict(W.ADAMW)
SENT = np.float32(np.uint32(0x7FB0B0B0).view(np.float32))


@pytest.mark.parametrize("n", [1, 7, 511, 512, 513, 4099, 65539, 1_000_003])
def test_conversion_matches_definition(n):
    say(f"blocked conversion n={n}")
    a, b, c = (W.np_f32_normal([80, k], n, 1.0) for k in range(3))
    st = Guarded(np.full(BL.blocked_state_len(n), SENT, dtype=np.float32))
    F.state_to_blocked(*(torch.from_numpy(x).cuda() for x in (a, b, c)), st.data(), n=n)
    torch.cuda.synchronize()
    assert bit_equal(st.data_host(), BL.to_blocked(a, b, c, fill=SENT))
    st.assert_guards("blocked state")
    back = [Guarded(np.full(n, SENT, dtype=np.float32)) for _ in range(3)]
    F.state_from_blocked(st.data(), *(g.data() for g in back), n=n)
    torch.cuda.synchronize()
    for g, want, what in zip(back, (a, b, c), ("master", "m", "v")):
        assert bit_equal(g.data_host(), want), what
        g.assert_guards(what)


def _layout(sizes, pad, wd, N, k):
    L, segs = F.shard_layout(sizes, N, k, pad, wd)
    lo, hi, osegs = OL.segments(sizes, pad, wd, N, k)
    flags = np.zeros(hi - lo, dtype=np.int64)
    for s in osegs:
        flags[s["shard_begin"]: s["shard_begin"] + s["length"]] = s["flags"]
    return L, segs, flags


CASES = [  # (n or layout, fan-in, phase d, clip)
    (1, 1, 0, 0.0), (513, 3, 5, 0.0), (2049, 8, 1, 0.0), (65539, 64, 7, 0.0),
    (300001, -1, 3, 0.0), (70003, 8, 2, 1e-3), (70003, -1, 6, 1e-3),
    (([5000, 3, 12000, 1, 7777, 40001], 16, [1, 0, 1, 1, 0, 1], 3, 1), 4, 4, 0.0),
    (([5000, 3, 12000, 1, 7777, 40001], 16, [1, 0, 1, 1, 0, 1], 3, 1), -1, 0, 10.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_blocked_step_matches_oracle_and_separate_layout(case):
    what, F_in, d, clip = CASES[case]
    if isinstance(what, int):
        n, lo = what, 1000 + d
        flags = np.full(n, OL.WEIGHT_DECAY, dtype=np.int64)
        sd, nseg = None, 0
    else:
        L, segs, flags = _layout(*what)
        n, lo = L.n, L.lo
        sd, nseg = F.segments_to_device(segs), L.n_segments
    real = (flags & OL.PADDING) == 0
    say(f"blocked step case {case}: n={n} F={F_in} d={d} clip={clip}")
    seed = 90 + case
    master0 = W.np_f32_normal([seed, 1], n, 0.02)
    m0 = W.np_f32_normal([seed, 2], n, 1e-3)
    v0 = (np.abs(W.np_f32_normal([seed, 3], n, 1e-3)) ** 2).astype(np.float32)
    blk = Guarded(BL.to_blocked(master0, m0, v0, fill=SENT))
    sep = [Guarded(master0), Guarded(m0), Guarded(v0)]
    flat_b = Guarded(np.zeros(n, np.uint16), pre=d)
    flat_s = Guarded(np.zeros(n, np.uint16), pre=d)
    om, omm, ov = master0.copy(), m0.copy(), v0.copy()
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in (1, 2):
        ohp = dict(HP)
        kw = dict(step=t, segs=sd, n_segments=nseg, flat_index0=lo - d, lo=lo, **HP)
        if F_in == -1:
            grad = W.np_f32_normal([seed, 10 + t], n, 1e-2)
            grad[~real] = np.nan
            gdev = torch.from_numpy(grad).cuda()
            if clip:
                F.grad_sumsq_shard(sumsq, grad=gdev, n=n, segs=sd, n_segments=nseg)
                ohp["grad_scale"] = float(OC.clipped_scale(OC.sumsq_exact(grad, real), clip))
                kw.update(max_grad_norm=clip, grad_sumsq=sumsq)
            F.adamw_shard_step_f32grad_blocked(blk.data(), gdev, n=n, flat=flat_b.window(), **kw)
            F.adamw_shard_step_f32grad(sep[0].data(), sep[1].data(), sep[2].data(), gdev,
                                       flat=flat_s.window(), **kw)
            om, omm, ov, oout = OS.shard_step_f32grad(om, omm, ov, grad, flags, ohp, t)
        else:
            contribs = [W.np_bf16_normal([seed, 20 + t, r], n, 1e-2) for r in range(F_in)]
            for cb in contribs:
                cb[~real] = 0x7FC0
            dev = [to_dev16(cb) for cb in contribs]
            if clip:
                F.grad_sumsq_shard(sumsq, contribs=dev, n=n, segs=sd, n_segments=nseg)
                ohp["grad_scale"] = float(OC.clipped_scale(OC.grad_sumsq(contribs, real), clip))
                kw.update(max_grad_norm=clip, grad_sumsq=sumsq)
            F.adamw_shard_step_blocked(blk.data(), dev, n=n, flat=flat_b.window(), **kw)
            F.adamw_shard_step(sep[0].data(), sep[1].data(), sep[2].data(), dev,
                               flat=flat_s.window(), **kw)
            om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, ohp, t)
        torch.cuda.synchronize()
        gm, gmm, gv = BL.from_blocked(blk.data_host(), n)
        assert_f32(gm, om, f"master step {t}")
        assert_f32(gmm, omm, f"m step {t}")
        assert_f32(gv, ov, f"v step {t}")
        assert_bf16(flat_b.data_host(), oout, f"bf16 step {t}")
        for x, g in zip((gm, gmm, gv), sep):
            assert bit_equal(x, g.data_host())
        assert bit_equal(flat_b.data_host(), flat_s.data_host())
    # Unused slots of the last block are never touched.
    st = blk.data_host()
    tail = np.ones(st.size, bool)
    tail[np.nonzero(BL.to_blocked(np.zeros(n, np.float32), np.zeros(n, np.float32),
                                  np.zeros(n, np.float32), fill=1.0) == 0.0)] = False
    assert (st[tail].view(np.uint32) == np.uint32(0x7FB0B0B0)).all()
    blk.assert_guards("blocked state")
    flat_b.assert_guards("flat window")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dense7b_n8_rank0", "dense70b_n64_rank0"])
def test_full_size_blocked_equals_separate(name):
    w = W.WORKLOADS[name]
    L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    n, lo = L.n, L.lo
    say(f"blocked full size {name} n={n}")
    dev = torch.device("cuda")
    sd = F.segments_to_device(segs, dev)
    master, m, v = W.torch_state(w, n, 0, dev)
    state = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device=dev)
    F.state_to_blocked(master, m, v, state)
    grads = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(w.fan_in)]
    flat_s = torch.empty(n, dtype=torch.int16, device=dev)
    flat_b = torch.empty(n, dtype=torch.int16, device=dev)
    for t in (1, 2):
        W.torch_grads_into(w, grads, t, 0)
        F.adamw_shard_step(master, m, v, grads, step=t, segs=sd, n_segments=L.n_segments,
                           flat=flat_s, flat_index0=lo, lo=lo, **w.hp)
        F.adamw_shard_step_blocked(state, grads, step=t, n=n, segs=sd, n_segments=L.n_segments,
                                   flat=flat_b, flat_index0=lo, lo=lo, **w.hp)
    back = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3)]
    F.state_from_blocked(state, *back)
    torch.cuda.synchronize()
    for x, y, what in zip(back, (master, m, v), ("master", "m", "v")):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), what
    assert torch.equal(flat_b, flat_s)
