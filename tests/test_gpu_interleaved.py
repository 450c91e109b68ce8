"""GPU parity of the interleaved gradient layout.

* grads_to_interleaved against the tests' definition of the layout, bit for bit, with the
  positions past n in the last block and the guard bands untouched;
* adamw_shard_step_interleaved against the oracle (fp32 state within relative 1e-5, bf16 within
  1 ulp) and bit for bit against adamw_shard_step_blocked on the same contributions, over sizes
  with ragged tails, the compile-time fan-ins 1, 2, 4 and 8 and run-time fan-ins, segment tables
  with NaN padding gradients, output phases and clipping; the gradient array is never written;
* grad_sumsq_shard_interleaved within relative 1e-12 of the oracle's exactly rounded sum and bit
  for bit equal to grad_sumsq_shard on the separate contributions (whole tiles, ragged tails,
  padding inside whole tiles, compile-time and run-time fan-ins); the clipped cases of the step
  take their norm from it;
* reduce_shard_interleaved and reduce_shard_sumsq_interleaved (plain and accumulating) bit for
  bit equal to the oracle's reduction and to the separate-array calls, the fused sum within
  relative 1e-12 of the oracle's exact sum and equal to the separate-array one;
* a ragged slice whose interleaved offsets pass 2^31 elements, and the 7B-shaped slice at full
  size: interleaved steps and sums equal the separate-contribution ones bit for bit.
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
from gpu_helpers import SENT16, Guarded, assert_bf16, assert_f32, bit_equal, say, to_dev16

pytestmark = pytest.mark.gpu
HP = dict(W.ADAMW)
SENT = np.float32(np.uint32(0x7FB0B0B0).view(np.float32))
SUMSQ_RTOL = 1e-12


@pytest.mark.parametrize("n", [1, 7, 511, 512, 513, 4099, 65539, 1_000_003])
@pytest.mark.parametrize("fan_in", [1, 3, 8])
def test_conversion_matches_definition(n, fan_in):
    say(f"interleave conversion n={n} F={fan_in}")
    contribs = [W.np_bf16_normal([81, fan_in, r], n, 1.0) for r in range(fan_in)]
    dst = Guarded(np.full(BL.interleaved_len(fan_in, n), SENT16, dtype=np.uint16))
    F.grads_to_interleaved([to_dev16(c) for c in contribs], dst.data(), n=n)
    torch.cuda.synchronize()
    assert np.array_equal(dst.data_host(), BL.to_interleaved(contribs, fill=SENT16))
    dst.assert_guards("interleaved gradients")


def _layout(sizes, pad, wd, N, k):
    L, segs = F.shard_layout(sizes, N, k, pad, wd)
    lo, hi, osegs = OL.segments(sizes, pad, wd, N, k)
    flags = np.zeros(hi - lo, dtype=np.int64)
    for s in osegs:
        flags[s["shard_begin"]: s["shard_begin"] + s["length"]] = s["flags"]
    return L, segs, flags


SMALL = ([5000, 3, 12000, 1, 7777, 40001], 16, [1, 0, 1, 1, 0, 1], 3, 1)
CASES = [  # (n or layout, fan-in, phase d, clip)
    (1, 1, 0, 0.0), (513, 3, 5, 0.0), (2049, 8, 1, 0.0), (65539, 64, 7, 0.0),
    (300001, 2, 3, 0.0), (40000, 4, 6, 0.0), (70003, 8, 2, 1e-3), (9000, 5, 0, 0.0),
    (SMALL, 4, 4, 0.0), (SMALL, 8, 0, 10.0), (SMALL, 1, 2, 0.0), (SMALL, 6, 7, 0.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_interleaved_step_matches_oracle_and_blocked_step(case):
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
    say(f"interleaved step case {case}: n={n} F={F_in} d={d} clip={clip}")
    seed = 190 + case
    master0 = W.np_f32_normal([seed, 1], n, 0.02)
    m0 = W.np_f32_normal([seed, 2], n, 1e-3)
    v0 = (np.abs(W.np_f32_normal([seed, 3], n, 1e-3)) ** 2).astype(np.float32)
    blk_i = Guarded(BL.to_blocked(master0, m0, v0, fill=SENT))
    blk_b = Guarded(BL.to_blocked(master0, m0, v0, fill=SENT))
    flat_i = Guarded(np.zeros(n, np.uint16), pre=d)
    flat_b = Guarded(np.zeros(n, np.uint16), pre=d)
    om, omm, ov = master0.copy(), m0.copy(), v0.copy()
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in (1, 2):
        ohp = dict(HP)
        kw = dict(step=t, n=n, segs=sd, n_segments=nseg, flat_index0=lo - d, lo=lo, **HP)
        contribs = [W.np_bf16_normal([seed, 20 + t, r], n, 1e-2) for r in range(F_in)]
        for cb in contribs:
            cb[~real] = 0x7FC0
        dev = [to_dev16(cb) for cb in contribs]
        packed = BL.to_interleaved(contribs, fill=SENT16)
        gi = Guarded(packed)
        kw_b = dict(kw)
        if clip:
            sumsq_b = torch.zeros(1, dtype=torch.float64, device="cuda")
            F.grad_sumsq_shard_interleaved(sumsq, gi.data(), F_in, n, segs=sd, n_segments=nseg)
            F.grad_sumsq_shard(sumsq_b, contribs=dev, n=n, segs=sd, n_segments=nseg)
            exact = OC.grad_sumsq(contribs, real)
            torch.cuda.synchronize()
            assert float(sumsq.item()) == float(sumsq_b.item())
            assert abs(float(sumsq.item()) - exact) <= SUMSQ_RTOL * exact
            ohp["grad_scale"] = float(OC.clipped_scale(exact, clip))
            kw.update(max_grad_norm=clip, grad_sumsq=sumsq)
            kw_b.update(max_grad_norm=clip, grad_sumsq=sumsq_b)
        F.adamw_shard_step_interleaved(blk_i.data(), gi.data(), F_in, flat=flat_i.window(), **kw)
        F.adamw_shard_step_blocked(blk_b.data(), dev, flat=flat_b.window(), **kw_b)
        om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, ohp, t)
        torch.cuda.synchronize()
        gm, gmm, gv = BL.from_blocked(blk_i.data_host(), n)
        assert_f32(gm, om, f"master step {t}")
        assert_f32(gmm, omm, f"m step {t}")
        assert_f32(gv, ov, f"v step {t}")
        assert_bf16(flat_i.data_host(), oout, f"bf16 step {t}")
        assert bit_equal(blk_i.data_host(), blk_b.data_host())
        assert bit_equal(flat_i.data_host(), flat_b.data_host())
        assert np.array_equal(gi.data_host(), packed), "gradient array written"
        gi.assert_guards("interleaved gradients")
    blk_i.assert_guards("blocked state")
    flat_i.assert_guards("flat window")


SUMSQ_CASES = [(1, 1), (7, 8), (513, 3), (32768, 4), (32769, 8), (1_000_003, 8), (2_500_001, 1),
               (300_017, 5), (100_003, 16), (70_001, 2)]


@pytest.mark.parametrize("n,F_in", SUMSQ_CASES)
def test_interleaved_sumsq_matches_exact_and_separate(n, F_in):
    say(f"interleaved sumsq n={n} F={F_in}")
    contribs = [W.np_bf16_normal([64, F_in, r], n, 1e-2) for r in range(F_in)]
    gi = Guarded(BL.to_interleaved(contribs, fill=SENT16))
    got_t = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    sep_t = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    F.grad_sumsq_shard_interleaved(got_t, gi.data(), F_in, n, scale=0.5)
    F.grad_sumsq_shard(sep_t, contribs=[to_dev16(c) for c in contribs], n=n, scale=0.5)
    torch.cuda.synchronize()
    got, sep = float(got_t.item()), float(sep_t.item())
    want = OC.grad_sumsq(contribs, np.ones(n, bool), 0.5)
    assert got == sep, (got, sep)
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)
    gi.assert_guards("interleaved gradients")


@pytest.mark.parametrize("F_in", [1, 3, 4, 8])
def test_interleaved_sumsq_padding_inside_whole_tiles(F_in):
    # 300 small tensors padded to 16, NaN in the padding, across many whole tiles.
    sizes = [(i * 7919) % 3001 + 1 for i in range(300)]
    L, segs, flags = _layout(sizes, 16, None, 2, 1)
    n = L.n
    real = (flags & OL.PADDING) == 0
    say(f"interleaved sumsq padded tiles F={F_in} n={n}")
    contribs = [W.np_bf16_normal([69, F_in, r], n, 1e-2) for r in range(F_in)]
    for c in contribs:
        c[~real] = 0x7FC0
    sd = F.segments_to_device(segs)
    got_t = torch.zeros(1, dtype=torch.float64, device="cuda")
    sep_t = torch.zeros(1, dtype=torch.float64, device="cuda")
    F.grad_sumsq_shard_interleaved(got_t, to_dev16(BL.to_interleaved(contribs)), F_in, n, segs=sd,
                                   n_segments=L.n_segments)
    F.grad_sumsq_shard(sep_t, contribs=[to_dev16(c) for c in contribs], n=n, segs=sd,
                       n_segments=L.n_segments)
    torch.cuda.synchronize()
    want = OC.grad_sumsq(contribs, real)
    assert float(got_t.item()) == float(sep_t.item())
    assert abs(float(got_t.item()) - want) <= SUMSQ_RTOL * want


RED_CASES = [(1, 1, False), (7, 3, True), (4099, 8, False), (32769, 8, True), (65539, 2, True),
             (300_017, 5, False), (1_000_003, 4, True), (300_017, 8, True), (98_304, 4, False),
             (70_001, 16, True)]


@pytest.mark.parametrize("n,F_in,acc", RED_CASES)
def test_interleaved_reductions_match_oracle_and_separate(n, F_in, acc):
    say(f"interleaved reduce n={n} F={F_in} accumulate={acc}")
    contribs = [W.np_bf16_normal([72, F_in, r], n, 1e-2) for r in range(F_in)]
    dev = [to_dev16(c) for c in contribs]
    gi = Guarded(BL.to_interleaved(contribs, fill=SENT16))
    acc0 = W.np_f32_normal([73, n], n, 1e-3) if acc else np.full(n, np.nan, np.float32)
    want = OS.accumulate_fp32(acc0, contribs, 0.5) if acc else OS.reduce_contributions(contribs, 0.5)
    # the plain and the accumulating reduction
    out_i, out_s = Guarded(acc0), Guarded(acc0)
    F.reduce_shard_interleaved(gi.data(), F_in, out_i.data(), accumulate=acc, scale=0.5)
    if acc:
        F.reduce_shard_accumulate(dev, out_s.data(), scale=0.5)
    else:
        F.reduce_shard(dev, out_s.data(), scale=0.5)
    torch.cuda.synchronize()
    assert bit_equal(out_i.data_host(), want)
    assert bit_equal(out_i.data_host(), out_s.data_host())
    out_i.assert_guards("out")
    # fused with the sum of squares
    sq_out_i, sq_out_s = Guarded(acc0), Guarded(acc0)
    res_i = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    res_s = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    F.reduce_shard_sumsq_interleaved(gi.data(), F_in, sq_out_i.data(), res_i, accumulate=acc,
                                     scale=0.5)
    F.reduce_shard_sumsq(dev, sq_out_s.data(), res_s, accumulate=acc, scale=0.5)
    torch.cuda.synchronize()
    assert bit_equal(sq_out_i.data_host(), want)
    sq_out_i.assert_guards("out")
    got, sep = float(res_i.item()), float(res_s.item())
    osum = OC.sumsq_exact(want)
    assert got == sep, (got, sep)
    assert abs(got - osum) <= SUMSQ_RTOL * osum, (got, osum)
    assert np.array_equal(gi.data_host(), BL.to_interleaved(contribs, fill=SENT16))
    gi.assert_guards("interleaved gradients")


@pytest.mark.parametrize("F_in,acc", [(8, False), (8, True), (4, True), (1, False), (3, True)])
def test_interleaved_reduce_sumsq_padding_inside_whole_tiles(F_in, acc):
    sizes = [(i * 7919) % 3001 + 1 for i in range(300)]
    L, segs, flags = _layout(sizes, 16, None, 2, 1)
    n = L.n
    real = (flags & OL.PADDING) == 0
    say(f"interleaved reduce+sumsq padded tiles F={F_in} accumulate={acc} n={n}")
    contribs = [W.np_bf16_normal([76, F_in, r], n, 1e-2) for r in range(F_in)]
    for c in contribs:
        c[~real] = 0x7FC0
    acc0 = W.np_f32_normal([77, n], n, 1e-3) if acc else np.zeros(n, np.float32)
    out = Guarded(acc0)
    res = torch.zeros(1, dtype=torch.float64, device="cuda")
    F.reduce_shard_sumsq_interleaved(to_dev16(BL.to_interleaved(contribs)), F_in, out.data(), res,
                                     accumulate=acc, scale=0.25, segs=F.segments_to_device(segs),
                                     n_segments=L.n_segments)
    torch.cuda.synchronize()
    want = (OS.accumulate_fp32(acc0, contribs, 0.25) if acc
            else OS.reduce_contributions(contribs, 0.25))
    assert bit_equal(out.data_host()[real], want[real])
    osum = OC.sumsq_exact(want, real)
    got = float(res.item())
    assert abs(got - osum) <= SUMSQ_RTOL * osum, (got, osum)


def _bf16_like(n, gen, std):
    return (torch.randn(n, generator=gen, device="cuda") * std).to(torch.bfloat16).view(torch.int16)


def _interleaved_equals_blocked(n, fan_in, segs_dev, n_segments, hp, state0_seed, steps=2):
    """Two steps through both calls on the same device inputs; returns nothing, asserts bits."""
    gen = torch.Generator(device="cuda").manual_seed(state0_seed)
    master = torch.randn(n, generator=gen, device="cuda") * 0.02
    m = torch.randn(n, generator=gen, device="cuda") * 1e-3
    v = (torch.randn(n, generator=gen, device="cuda") * 1e-3) ** 2
    st_i = torch.empty(F.state_blocked_elems(n), dtype=torch.float32, device="cuda")
    F.state_to_blocked(master, m, v, st_i)
    st_b = st_i.clone()
    del master, m, v
    grads = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(fan_in)]
    gi = torch.empty(F.grads_interleaved_elems(fan_in, n), dtype=torch.int16, device="cuda")
    flat_i = torch.empty(n, dtype=torch.int16, device="cuda")
    flat_b = torch.empty(n, dtype=torch.int16, device="cuda")
    sq_i = torch.zeros(1, dtype=torch.float64, device="cuda")
    sq_b = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in range(1, steps + 1):
        for g in grads:
            g.copy_(_bf16_like(n, gen, 1e-3))
        F.grads_to_interleaved(grads, gi, n=n)
        F.grad_sumsq_shard_interleaved(sq_i, gi, fan_in, n, segs=segs_dev, n_segments=n_segments)
        F.grad_sumsq_shard(sq_b, contribs=grads, n=n, segs=segs_dev, n_segments=n_segments)
        kw = dict(step=t, n=n, segs=segs_dev, n_segments=n_segments, flat_index0=0, lo=0, **hp)
        F.adamw_shard_step_interleaved(st_i, gi, fan_in, flat=flat_i, **kw)
        F.adamw_shard_step_blocked(st_b, grads, flat=flat_b, **kw)
        torch.cuda.synchronize()
        assert torch.equal(st_i.view(torch.int32), st_b.view(torch.int32)), f"state step {t}"
        assert torch.equal(flat_i, flat_b), f"bf16 step {t}"
        assert float(sq_i.item()) == float(sq_b.item()), f"sum of squares step {t}"
        say(f"  step {t} ok")
    del st_i, st_b, flat_i, flat_b
    red_i = torch.empty(n, dtype=torch.float32, device="cuda")
    red_b = torch.empty(n, dtype=torch.float32, device="cuda")
    F.reduce_shard_interleaved(gi, fan_in, red_i, n=n)
    F.reduce_shard(grads, red_b, n=n)
    F.reduce_shard_interleaved(gi, fan_in, red_i, accumulate=True, scale=0.5, n=n)
    F.reduce_shard_accumulate(grads, red_b, scale=0.5, n=n)
    torch.cuda.synchronize()
    assert torch.equal(red_i.view(torch.int32), red_b.view(torch.int32)), "reduction"
    del red_i, red_b, grads, gi
    torch.cuda.empty_cache()


def test_interleaved_offsets_beyond_2_31():
    """Fan-in 8 on a ragged slice of 2^28 + 123 elements: the interleaved array holds
    8 * (2^28 + 512) elements, so its offsets pass 2^31; the conversion, two steps, their sums
    of squares and a plain and an accumulating reduction equal the separate-contribution calls
    bit for bit over the whole slice."""
    n = (1 << 28) + 123
    say(f"interleaved offsets beyond 2^31: n={n}")
    assert F.grads_interleaved_elems(8, n) > (1 << 31)
    L, segs = F.shard_layout([n], 1, 0)
    _interleaved_equals_blocked(n, 8, F.segments_to_device(segs), L.n_segments, HP, 7)


@pytest.mark.slow
def test_full_size_interleaved_equals_blocked():
    w = W.WORKLOADS["dense7b_n8_rank0"]
    L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
    say(f"interleaved full size dense7b_n8_rank0 n={L.n}")
    assert L.lo == 0
    _interleaved_equals_blocked(L.n, w.fan_in, F.segments_to_device(segs), L.n_segments, w.hp, 8)
