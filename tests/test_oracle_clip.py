"""Pins for the oracle's sharded gradient norm, clip coefficient and fp32 accumulation.

* sum of squares -- closed forms, exact rational arithmetic, and a library routine (PyTorch's
  float64 vector norm);
* the sharded norm -- the ranks' parts add up to the norm of the whole gradient and each rank's
  own part is never larger (a local norm underestimates the global one, as the clipping passage
  of "FSDP: Fully Sharded Data Parallel Training at Scale" points out);
* the clip coefficient -- PyTorch's clip_grad_norm_ run in float64 on the whole gradient;
* fp32 accumulation -- exact integer sums, and the accumulate-then-step path equals the fused
  step when there is a single micro-batch.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import clip, layout
from oracle.bf16 import f32_to_bf16_rne
from oracle.step import (accumulate_fp32, reduce_contributions, shard_step, shard_step_f32grad)

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def bf(x):
    return f32_to_bf16_rne(np.asarray(x, dtype=np.float32))


def test_sumsq_closed_forms():
    assert clip.sumsq_exact(np.full(1000, 3.0, np.float32)) == 9000.0
    assert clip.sumsq_exact(np.float32([3.0, 4.0])) == 25.0
    assert clip.sumsq_exact(np.zeros(7, np.float32)) == 0.0
    # padding does not count
    g = np.float32([1.0, 2.0, 100.0])
    assert clip.sumsq_exact(g, [True, True, False]) == 5.0


def test_sumsq_exact_rational():
    rng = np.random.default_rng(1)
    g = (rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)).astype(np.float32)
    exact = sum(Fraction(float(x)) ** 2 for x in g)
    assert clip.sumsq_exact(g) == float(exact)          # one rounding of the exact sum


def test_sumsq_against_library_norm():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(200_000).astype(np.float32) * np.float32(1e-3)
    lib = torch.linalg.vector_norm(torch.from_numpy(g).double()).item()
    assert abs(np.sqrt(clip.sumsq_exact(g)) - lib) <= 1e-13 * lib


@pytest.mark.parametrize("N", [1, 2, 3, 8, 16])
def test_shard_parts_add_up_and_underestimate(N):
    rng = np.random.default_rng(3 + N)
    sizes = [int(s) for s in rng.integers(1, 3000, 12)]
    wd = [bool(x) for x in rng.random(12) < 0.5]
    offs, P = layout.flatten_offsets(sizes, 16)
    F = 4
    full = [bf(rng.standard_normal(P) * 1e-2) for _ in range(F)]
    flags_full = np.zeros(P, dtype=np.int64)
    for k in range(N):
        lo, hi, segs = layout.segments(sizes, 16, wd, N, k)
        for sg in segs:
            flags_full[lo + sg["shard_begin"]: lo + sg["shard_begin"] + sg["length"]] = sg["flags"]
    real_full = (flags_full & layout.PADDING) == 0
    whole = clip.grad_sumsq(full, real_full)
    parts = []
    for k in range(N):
        lo, hi, _ = layout.segments(sizes, 16, wd, N, k)
        part = clip.grad_sumsq([c[lo:hi] for c in full], real_full[lo:hi])
        assert part <= whole
        parts.append(part)
    assert abs(sum(parts) - whole) <= N * 2.0 ** -52 * whole
    if N > 1:
        assert max(parts) < whole


@pytest.mark.parametrize("max_norm", [1e-4, 0.05, 1.0, 1e6])
def test_clip_coefficient_against_library(max_norm):
    rng = np.random.default_rng(4)
    sizes = [300, 17, 4000, 1]
    grads = [rng.standard_normal(s).astype(np.float32) * np.float32(1e-2) for s in sizes]
    params = [torch.nn.Parameter(torch.zeros(s, dtype=torch.float64)) for s in sizes]
    for p, g in zip(params, grads):
        p.grad = torch.from_numpy(g.astype(np.float64))
    total = torch.nn.utils.clip_grad_norm_(params, max_norm, norm_type=2.0, foreach=False).item()
    sumsq = clip.sumsq_exact(np.concatenate(grads))
    assert abs(np.sqrt(sumsq) - total) <= 1e-14 * total
    coef = clip.clip_coefficient(sumsq, max_norm)
    for p, g in zip(params, grads):
        ratio = p.grad.numpy() / g.astype(np.float64)
        assert np.allclose(ratio, coef, rtol=1e-14, atol=0)
    assert 0.0 < coef <= 1.0
    assert (coef == 1.0) == (max_norm >= np.sqrt(sumsq) + clip.CLIP_EPS)


def test_clipped_scale_rounds_once():
    s = clip.clipped_scale(4.0, 1.0, grad_scale=0.5)     # coef = 1/(2+1e-6)
    assert s == np.float32(0.5 * (1.0 / (2.0 + 1e-6)))
    assert clip.clipped_scale(1e-12, 1.0) == np.float32(1.0)


def test_accumulate_integer_sums():
    rng = np.random.default_rng(5)
    acc = np.zeros(1000, np.float32)
    total = np.zeros(1000, np.int64)
    for mb in range(7):
        vals = rng.integers(-100, 101, size=(3, 1000))
        acc = accumulate_fp32(acc, [bf(v) for v in vals])
        total += vals.sum(axis=0)
    assert np.array_equal(acc, total.astype(np.float32))
    acc2 = accumulate_fp32(np.ones(4, np.float32), [bf([2.0, 4.0, 6.0, 8.0])], scale=0.5)
    assert np.array_equal(acc2, np.float32([2.0, 3.0, 4.0, 5.0]))


def test_single_microbatch_accumulation_matches_fused_step():
    rng = np.random.default_rng(6)
    n = 5000
    flags = np.where(rng.random(n) < 0.1, layout.WEIGHT_DECAY | layout.PADDING, layout.WEIGHT_DECAY)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    contribs = [bf(rng.standard_normal(n) * 1e-2) for _ in range(8)]
    a = shard_step(master, m, v, contribs, flags, HP, 4)
    acc = accumulate_fp32(np.zeros(n, np.float32), contribs)
    b = shard_step_f32grad(master, m, v, acc, flags, HP, 4)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()


def test_accumulation_differs_from_bf16_accumulation():
    # Accumulating in float32 keeps contributions that a bf16 accumulator would round away.
    big, small = bf([256.0])[0], bf([1.0])[0]
    acc = np.zeros(1, np.float32)
    for c in [big] + [small] * 4:
        acc = accumulate_fp32(acc, [np.array([c], np.uint16)])
    assert acc[0] == np.float32(260.0)
    acc16 = np.zeros(1, np.float32)
    for c in [big] + [small] * 4:                          # re-rounded to bf16 after every add
        acc16 = np.asarray(reduce_contributions([bf(acc16), np.array([c], np.uint16)]))
    assert float(reduce_contributions([bf(acc16)])[0]) == 256.0
