"""GPU parity of the C-ABI calls against the oracle, at sizes the oracle finishes in seconds.

Every case runs through the library (ctypes binding -> libfsdpshard.so -> gfx950 kernels) and is
compared with the oracle on the same seeded inputs, element by element:
  fp32 master / m / v within relative 1e-5, bf16 params within 1 ulp (NaN matches NaN).
Every written buffer carries sentinel guard bands (and the flat window a guarded prefix before
the slice) that must survive untouched.  Sizes span several 512-element wave groups and
2048-element work-group rounds plus ragged tails; the bf16 destination is exercised at all eight
2-byte phases; segment tables cover padding, weight-decay masks and one-element runs.
"""

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from oracle import layout as OL
from oracle import step as OS
from oracle.bf16 import f32_to_bf16_rne
from gpu_helpers import (Guarded, assert_bf16, assert_f32, bit_equal, say, to_dev16)

pytestmark = pytest.mark.gpu
HP = dict(W.ADAMW)


def _layout_case(sizes, pad, wd, N, k):
    L, segs = F.shard_layout(sizes, N, k, pad, wd)
    lo, hi, osegs = OL.segments(sizes, pad, wd, N, k)
    assert (L.lo, L.hi) == (lo, hi)
    flags = np.zeros(hi - lo, dtype=np.int64)
    for s in osegs:
        flags[s["shard_begin"]: s["shard_begin"] + s["length"]] = s["flags"]
    return L, segs, flags


def run_case(n=None, F_in=8, steps=2, d=0, layout=None, seed=0, warm_state=True, nan_pad=False,
             hp=HP, grad_std=1e-2, check_bitexact=False, lo=1000):
    """Run `steps` fused steps on one slice through the library and through the oracle."""
    if layout is not None:
        L, segs, flags = _layout_case(*layout)
        n, lo = L.n, L.lo
        segs_dev = F.segments_to_device(segs) if L.n_segments else None
        nseg = L.n_segments
    else:
        flags = np.full(n, OL.WEIGHT_DECAY, dtype=np.int64)
        segs_dev, nseg = None, 0
    say(f"case n={n} F={F_in} steps={steps} d={d} segs={nseg} seed={seed}")
    master0 = W.np_f32_normal([seed, 1], n, 0.02)
    if warm_state:
        m0 = W.np_f32_normal([seed, 2], n, 1e-3)
        v0 = np.abs(W.np_f32_normal([seed, 3], n, 1e-3)) ** 2
        v0 = v0.astype(np.float32)
    else:
        m0 = np.zeros(n, np.float32)
        v0 = np.zeros(n, np.float32)
    gm, gmm, gv = Guarded(master0), Guarded(m0), Guarded(v0)
    flat = Guarded(np.zeros(n, np.uint16), pre=d)
    om, omm, ov = master0.copy(), m0.copy(), v0.copy()
    for t in range(1, steps + 1):
        contribs = [W.np_bf16_normal([seed, 100 + t, r], n, grad_std) for r in range(F_in)]
        if nan_pad:
            for c in contribs:
                c[(flags & OL.PADDING) != 0] = 0x7FC0
        dev = [to_dev16(c) for c in contribs]
        F.adamw_shard_step(gm.data(), gmm.data(), gv.data(), dev, step=t, segs=segs_dev,
                           n_segments=nseg, flat=flat.window(), flat_index0=lo - d, lo=lo,
                           **hp)
        torch.cuda.synchronize()
        om, omm, ov, oout = OS.shard_step(om, omm, ov, contribs, flags, hp, t)
        assert_f32(gm.data_host(), om, f"master step {t}")
        assert_f32(gmm.data_host(), omm, f"m step {t}")
        assert_f32(gv.data_host(), ov, f"v step {t}")
        assert_bf16(flat.data_host(), oout, f"bf16 step {t}")
        if check_bitexact:
            assert bit_equal(gm.data_host(), om) and bit_equal(gmm.data_host(), omm)
            assert bit_equal(gv.data_host(), ov) and bit_equal(flat.data_host(), oout)
    for g, what in ((gm, "master"), (gmm, "m"), (gv, "v"), (flat, "flat window")):
        g.assert_guards(what)


SIZES = [1, 5, 8, 9, 63, 64, 511, 512, 513, 2047, 2048, 2049, 4103, 8191, 65539, 300001]
FANS = [1, 2, 3, 4, 5, 8, 16, 64]


@pytest.mark.parametrize("i", range(len(SIZES)))
def test_step_sizes_and_fanins(i):
    n = SIZES[i]
    run_case(n=n, F_in=FANS[i % len(FANS)], d=(3 * i) % 8, steps=2, seed=i)


@pytest.mark.parametrize("d", range(32))
@pytest.mark.parametrize("F_in", [1, 8, 3])
def test_every_output_phase(d, F_in):
    # d elements between the 128-byte aligned guard and the window: every phase of the slice
    # start against a 16-byte vector and a 64-byte line; 6151 elements are three whole
    # work-groups (the bf16 edge exchange) and a tail
    run_case(n=6151, F_in=F_in, d=d, steps=2, seed=40 + d)


@pytest.mark.parametrize("d", range(32))
@pytest.mark.parametrize("F_in", [1, 8])
def test_every_output_phase_with_a_partial_last_work_group(d, F_in):
    # 5157 elements: two whole work-groups (which exchange bf16 edge words through LDS), then a
    # work-group whose first two groups are whole and whose third holds the slice's last 37
    # elements, so its whole groups store their edges without the exchange
    run_case(n=5157, F_in=F_in, d=d, steps=2, seed=90 + d)


@pytest.mark.parametrize("F_in", [1, 3, 8])
def test_many_groups_and_edges(F_in):
    # hundreds of work-groups (the XCD tile map's whole blocks and identity tail), a ragged last
    # group, and a segment table with tiny tensors and NaN padding gradients
    run_case(n=300_017, F_in=F_in, d=5, steps=1, seed=7)
    run_case(layout=([5000, 3, 12000, 1, 1, 1, 7777, 100000], 16, [1, 0, 1, 1, 0, 1, 0, 1], 3, 1),
             F_in=F_in, steps=1, seed=8, nan_pad=True)


def test_bitexact_representative():
    run_case(n=300001, F_in=8, d=1, steps=3, seed=3, check_bitexact=True)
    run_case(n=70001, F_in=3, d=6, steps=2, seed=4, check_bitexact=True,
             layout=([3000, 17, 1, 40000, 5, 26000, 999], 16, [1, 0, 1, 1, 0, 1, 0], 3, 1))


@pytest.mark.parametrize("case", [
    ([100, 7, 1, 33, 16, 2, 90], 16, [1, 0, 1, 1, 0, 1, 0], 1, 0),     # whole flat vector
    ([100, 7, 1, 33, 16, 2, 90], 16, [1, 0, 1, 1, 0, 1, 0], 3, 2),
    ([1] * 300, 4, [i % 3 == 0 for i in range(300)], 2, 1),           # 1-element runs
    ([5000, 3, 12000, 1, 1, 1, 7777], 8, None, 5, 3),
    ([4096 * 4 + 3] * 5, 16, [0, 1, 0, 1, 0], 7, 6),
])
def test_segment_tables(case):
    run_case(layout=case, F_in=4, steps=2, seed=11, nan_pad=True)


def test_no_decay_and_grad_scale():
    hp = dict(HP, weight_decay=0.0, grad_scale=0.125)
    run_case(n=20011, F_in=8, d=2, steps=2, hp=hp, seed=12)
    run_case(n=20011, F_in=2, d=0, steps=2, hp=dict(HP, grad_scale=3.0), seed=13)


def test_first_step_from_zero_state():
    run_case(n=30001, F_in=8, d=4, steps=1, seed=14, warm_state=False)


def test_special_values_propagate():
    # Inf, NaN, huge and denormal gradients in real elements, and denormal / huge state values
    n = 4096 + 77
    run_case(n=n, F_in=1, steps=1, seed=15)
    rng = np.random.default_rng(15)
    master = W.np_f32_normal([15, 1], n, 0.02)
    master[:8] = np.float32([1e-40, -1e-40, 3e38, -3e38, 0.0, -0.0, 1e-45, np.inf])
    m0 = np.zeros(n, np.float32)
    v0 = np.zeros(n, np.float32)
    c = W.np_bf16_normal([15, 9], n, 1e-2)
    c[8:16] = [0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x0000]
    c2 = W.np_bf16_normal([15, 10], n, 1e-2)
    c2[8:16] = [0xFF80, 0x0000, 0x0000, 0x0001, 0x0001, 0x7F7F, 0x7F7F, 0x8000]
    gm, gmm, gv = Guarded(master), Guarded(m0), Guarded(v0)
    flat = Guarded(np.zeros(n, np.uint16), pre=3)
    F.adamw_shard_step(gm.data(), gmm.data(), gv.data(), [to_dev16(c), to_dev16(c2)], step=1,
                       flat=flat.window(), flat_index0=997, lo=1000, **HP)
    torch.cuda.synchronize()
    flags = np.full(n, OL.WEIGHT_DECAY)
    om, omm, ov, oout = OS.shard_step(master, m0, v0, [c, c2], flags, HP, 1)
    assert_f32(gm.data_host(), om, "master")
    assert_f32(gmm.data_host(), omm, "m")
    assert_f32(gv.data_host(), ov, "v")
    assert_bf16(flat.data_host(), oout, "bf16")
    assert np.isnan(om[8]) and np.isnan(gm.data_host()[8])        # Inf - Inf reaches the weight
    for g, what in ((gm, "master"), (gmm, "m"), (gv, "v"), (flat, "flat")):
        g.assert_guards(what)


def test_zero_length_is_a_no_op():
    flat = Guarded(np.zeros(0, np.uint16), pre=8)
    gm = Guarded(np.zeros(0, np.float32))
    c = torch.zeros(8, dtype=torch.int16, device="cuda")
    F.adamw_shard_step(gm.full[64:], gm.full[64:], gm.full[64:], [c], step=1, n=0,
                       flat=flat.window(), flat_index0=0, lo=8, **HP)
    torch.cuda.synchronize()
    flat.assert_guards("flat")
    gm.assert_guards("master")


def test_all_ranks_fill_the_flat_vector():
    """Every rank of P = 1,000,003 over N = 8 writes its slice into one shared flat bf16 vector;
    after each step the union equals the oracle's bf16 copy of the whole updated vector."""
    w = W.WORKLOADS["p1000003_n8_rank3"]
    P, N = w.total, w.world_size
    master_full, _, _ = W.np_state(w, P, 0)
    m_full = np.zeros(P, np.float32)
    v_full = np.zeros(P, np.float32)
    flat = Guarded(np.zeros(P, np.uint16))
    ranks = []
    for k in range(N):
        L, segs = F.shard_layout(w.sizes, N, k)
        ranks.append((L, Guarded(master_full[L.lo:L.hi]), Guarded(m_full[L.lo:L.hi]),
                      Guarded(v_full[L.lo:L.hi])))
    om, omm, ov = master_full.copy(), m_full.copy(), v_full.copy()
    flags = np.full(P, OL.WEIGHT_DECAY)
    for t in range(1, w.steps + 1):
        grads = W.np_grads(w, P, t, 0)
        for L, gm, gmm, gv in ranks:
            dev = [to_dev16(g[L.lo:L.hi]) for g in grads]
            F.adamw_shard_step(gm.data(), gmm.data(), gv.data(), dev, step=t, flat=flat.window(),
                               flat_index0=0, lo=L.lo, **w.hp)
        torch.cuda.synchronize()
        om, omm, ov, oout = OS.shard_step(om, omm, ov, grads, flags, w.hp, t)
        assert_bf16(flat.data_host(), oout, f"flat vector step {t}")
        for L, gm, gmm, gv in ranks:
            assert_f32(gm.data_host(), om[L.lo:L.hi], f"master rank lo={L.lo}")
            assert_f32(gv.data_host(), ov[L.lo:L.hi], f"v rank lo={L.lo}")
    flat.assert_guards("flat")
    for _, gm, gmm, gv in ranks:
        gm.assert_guards("master")


def test_deterministic_repeat():
    outs = []
    for rep in range(2):
        n = 125_000
        master = W.np_f32_normal([21, 1], n, 0.02)
        gm, gmm, gv = Guarded(master), Guarded(np.zeros(n, np.float32)), Guarded(np.zeros(n, np.float32))
        flat = Guarded(np.zeros(n, np.uint16), pre=1)
        for t in (1, 2, 3):
            dev = [to_dev16(W.np_bf16_normal([21, t, r], n, 1e-2)) for r in range(8)]
            F.adamw_shard_step(gm.data(), gmm.data(), gv.data(), dev, step=t, flat=flat.window(),
                               flat_index0=374_999, lo=375_000, **HP)
        torch.cuda.synchronize()
        outs.append([gm.host().tobytes(), gmm.host().tobytes(), gv.host().tobytes(),
                     flat.host().tobytes()])
    assert outs[0] == outs[1]


# ---------------------------------------------------------------------- standalone calls

@pytest.mark.parametrize("n,F_in,scale", [(1, 1, 1.0), (9, 3, 0.5), (2049, 8, 1.0),
                                          (65539, 64, 0.125), (300001, 5, 2.0)])
def test_reduce_shard(n, F_in, scale):
    say(f"reduce n={n} F={F_in}")
    contribs = [W.np_bf16_normal([31, r], n, 1e-2) for r in range(F_in)]
    out = Guarded(np.zeros(n, np.float32))
    F.reduce_shard([to_dev16(c) for c in contribs], out.data(), scale=scale)
    torch.cuda.synchronize()
    want = OS.reduce_contributions(contribs, scale)
    assert_f32(out.data_host(), want, "reduce")
    assert bit_equal(out.data_host(), want)
    out.assert_guards("reduce out")


def test_reduce_rank_order_fixture():
    # 1 + 2^-24 + 2^-24 is 1.0 in rank order (ties to even) and 1 + 2^-23 in any order that adds
    # the small terms first; the kernel must give the rank-order result.
    one, tiny = f32_to_bf16_rne(np.float32([1.0]))[0], f32_to_bf16_rne(np.float32([2.0 ** -24]))[0]
    n = 4099
    c = [np.full(n, one, np.uint16), np.full(n, tiny, np.uint16), np.full(n, tiny, np.uint16)]
    out = Guarded(np.zeros(n, np.float32))
    F.reduce_shard([to_dev16(x) for x in c], out.data())
    torch.cuda.synchronize()
    assert np.all(out.data_host() == np.float32(1.0))


@pytest.mark.parametrize("d", [0, 1, 4, 7])
@pytest.mark.parametrize("case", [None, ([100, 7, 1, 33, 16, 2, 90], 16, [1, 0, 1, 1, 0, 1, 0], 3, 1)])
def test_unflatten(d, case):
    if case is None:
        n, lo, segs_dev, nseg = 10007, 5000, None, 0
        flags = np.full(n, OL.WEIGHT_DECAY)
    else:
        L, segs, flags = _layout_case(*case)
        n, lo, nseg = L.n, L.lo, L.n_segments
        segs_dev = F.segments_to_device(segs)
    master = W.np_f32_normal([41, d], n, 0.02)
    master[::97] = np.float32(np.nan)
    gm = Guarded(master)
    flat = Guarded(np.zeros(n, np.uint16), pre=d)
    F.unflatten_bf16(gm.data(), flat.window(), flat_index0=lo - d, lo=lo, segs=segs_dev,
                     n_segments=nseg)
    torch.cuda.synchronize()
    want = OS.unflatten_bf16(master, (flags & OL.PADDING) == 0)
    assert_bf16(flat.data_host(), want, "unflatten")
    assert bit_equal(flat.data_host(), want)
    flat.assert_guards("flat")
    gm.assert_guards("master")


def test_errors_raise():
    x = torch.zeros(16, device="cuda")
    c = torch.zeros(16, dtype=torch.int16, device="cuda")
    with pytest.raises(F.FsdpShardError):
        F.adamw_shard_step(x[1:], x[1:], x[1:], [c], step=1, n=4, **HP)    # misaligned state
    with pytest.raises(F.FsdpShardError):
        F.adamw_shard_step(x, x, x, [c], step=1, n=4, **HP)                # aliasing state


def test_calibration_kernels():
    """The measurement aids do what their header says (they are not part of the step)."""
    n = 8 * 3001
    src = torch.arange(n * 4, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    F.stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    rng = np.random.default_rng(51)
    grads = [rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16) for _ in range(8)]
    st = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    dev_s = [torch.from_numpy(x.copy()).cuda() for x in st]
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    F.stream_mix([to_dev16(g) for g in grads], dev_s[0], dev_s[1], dev_s[2], out)
    torch.cuda.synchronize()
    words = np.stack([g.view(np.uint32) for g in grads]).reshape(8, -1, 4)
    x = np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=2), axis=0)   # per 8-element vector
    for k in range(3):
        want = st[k].view(np.uint32).reshape(-1, 8).copy()
        want[:, 0] ^= x
        assert np.array_equal(dev_s[k].cpu().numpy().view(np.uint32).reshape(-1, 8), want)
    o = out.cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.array_equal(o[:, 3], x)
    assert np.array_equal(o[:, 0], st[0].view(np.uint32).reshape(-1, 8)[:, 1])
