"""grad_sumsq_shard_noalloc, the call that allocates nothing (its partials live in the library's
own per-device array), against grad_sumsq_shard with a caller workspace: two calls in a row,
the second on a smaller slice, each bit-equal to the workspace call (same kernels, same fixed
order) and within relative 1e-12 of the oracle's exactly rounded sum of squares."""

import ctypes

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from oracle import clip as OC
from oracle import layout as OL
from gpu_helpers import say, to_dev16

pytestmark = pytest.mark.gpu


def _case(sizes, pad, wd, N, k, fan_in, seed, scale):
    """Inputs of one slice: bf16 contributions (fan_in >= 1, NaN in the padding) or one fp32
    gradient shard (fan_in 0), with the oracle's sum of squares."""
    L, segs = F.shard_layout(sizes, N, k, pad, wd)
    lo, hi, osegs = OL.segments(sizes, pad, wd, N, k)
    assert (L.lo, L.hi) == (lo, hi)
    n = L.n
    real = np.ones(n, dtype=bool)
    for s in osegs:
        if s["flags"] & OL.PADDING:
            real[s["shard_begin"]: s["shard_begin"] + s["length"]] = False
    if fan_in == 0:
        grad = W.np_f32_normal([seed, 1], n, 1e-2)
        grad[~real] = np.nan
        dev = dict(grad=torch.from_numpy(grad).cuda())
        want = OC.sumsq_exact(grad * np.float32(scale), real)
    else:
        contribs = [W.np_bf16_normal([seed, 2, r], n, 1e-2) for r in range(fan_in)]
        for c in contribs:
            c[~real] = 0x7FC0
        dev = dict(contribs=[to_dev16(c) for c in contribs])
        want = OC.grad_sumsq(contribs, real, scale)
    return n, L.n_segments, F.segments_to_device(segs), dev, want


def _both(n, nseg, sd, dev, scale, stream=None):
    """Sum of squares through the workspace call and through the allocation-free call."""
    ws = torch.empty(F.grad_sumsq_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    a = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    b = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    F.grad_sumsq_shard(a, n=n, scale=scale, segs=sd, n_segments=nseg, workspace=ws, stream=stream,
                       **dev)
    F.grad_sumsq_shard_noalloc(b, n=n, scale=scale, segs=sd, n_segments=nseg, stream=stream, **dev)
    torch.cuda.synchronize()
    return float(a.item()), float(b.item())


CASES = [
    # 3.3 M elements (101 partials), fan-in 8, padding and decay mask; then 70,001 elements
    # (3 partials) from an fp32 shard; then a 1,027-element slice (1 partial) at fan-in 3.
    dict(sizes=[1_000_003, 17, 2_300_000, 5], pad=16, wd=[1, 0, 1, 1], N=1, k=0, fan_in=8,
         seed=11, scale=1.0),
    dict(sizes=[50_000, 3, 90_000, 1], pad=8, wd=None, N=2, k=1, fan_in=0, seed=12, scale=0.5),
    dict(sizes=[1_000, 27], pad=1, wd=None, N=1, k=0, fan_in=3, seed=13, scale=2.0),
]


def test_noalloc_matches_workspace_call_two_calls_in_a_row():
    for i, c in enumerate(CASES):
        n, nseg, sd, dev, want = _case(c["sizes"], c["pad"], c["wd"], c["N"], c["k"], c["fan_in"],
                                       c["seed"], c["scale"])
        say(f"noalloc call {i}: n={n} fan_in={c['fan_in']} partials="
            f"{F.grad_sumsq_workspace_bytes(n) // 8}")
        a, b = _both(n, nseg, sd, dev, c["scale"])
        assert np.float64(a).view(np.uint64) == np.float64(b).view(np.uint64), (a, b)
        assert abs(b - want) <= 1e-12 * want, (b, want)


def test_noalloc_on_a_side_stream_after_a_larger_call():
    big = _case([4_000_037], 1, None, 1, 0, 4, 21, 1.0)
    small = _case([33_333], 1, None, 1, 0, 1, 22, 1.0)
    torch.cuda.synchronize()                 # inputs are in place before the side stream reads
    s = torch.cuda.Stream()
    for n, nseg, sd, dev, want in (big, small):
        say(f"noalloc side stream: n={n}")
        with torch.cuda.stream(s):
            a, b = _both(n, nseg, sd, dev, 1.0, stream=s)
        assert np.float64(a).view(np.uint64) == np.float64(b).view(np.uint64), (a, b)
        assert abs(b - want) <= 1e-12 * want, (b, want)


def test_noalloc_refuses_slices_beyond_its_array():
    # Checked before anything is launched: the length alone decides, no element is read.
    g = torch.zeros(8, dtype=torch.int16, device="cuda")
    out = torch.zeros(1, dtype=torch.float64, device="cuda")
    arr = (ctypes.c_void_p * 1)(g.data_ptr())
    f = F.lib().grad_sumsq_shard_noalloc
    assert f(arr, 1, None, F.NOALLOC_MAX_ELEMS + 1, None, 0, 1.0, out.data_ptr(), None) == 3
    assert f(arr, 1, None, 8, None, 0, 1.0, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert float(out.item()) == 0.0
