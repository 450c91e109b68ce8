"""Pins for the oracle's reduction and AdamW step.

What fixes each result (no pin re-types the oracle's own formula):
* reduction -- an order-sensitivity fixture whose rank-order fp32 result differs from any other
  order, exact sums of small integers (exact in fp32 whatever the order), the F = 1 widening,
  and the +0 start value.
* AdamW -- a library routine for the same definition (PyTorch's CPU AdamW run in float64, which
  applies the learning-rate-scaled decoupled decay and then the bias-corrected Adam step) over
  several steps, with a tolerance derived from float32 rounding; the closed forms of the first
  step from zero moments (each weight moves by about lr*sign(g)) and of a zero gradient (the
  moments only decay); padding leaves state bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import layout
from oracle.bf16 import bf16_to_f32, f32_to_bf16_rne
from oracle.step import (adamw_update, adamw_update_f64, hyper_constants, reduce_contributions,
                         shard_step)

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
U24 = 2.0 ** -24


def bf(x):
    return f32_to_bf16_rne(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- reduction

def test_rank_order_fixture():
    # 1 + 2^-24 is a tie in fp32 and rounds to even (1.0); summing the two small terms first gives
    # exactly 1 + 2^-23.  Only the rank order 0, 1, 2 from +0 produces 1.0.
    c = [bf([1.0]), bf([U24]), bf([U24])]
    assert float(bf16_to_f32(c[1])[0]) == U24              # 2^-24 is exact in bf16
    assert reduce_contributions(c)[0] == np.float32(1.0)
    assert reduce_contributions(c[::-1])[0] == np.float32(1.0 + 2.0 ** -23)


def test_exact_integer_sums():
    rng = np.random.default_rng(5)
    for F in (1, 2, 3, 8, 16, 64):
        vals = rng.integers(-128, 129, size=(F, 1000))   # all exact in bf16 (8 significant bits)
        c = [bf(v) for v in vals]
        assert np.array_equal(reduce_contributions(c), vals.sum(axis=0).astype(np.float32))


def test_single_contribution_is_the_widening():
    rng = np.random.default_rng(6)
    h = rng.integers(0, 1 << 16, 100000, dtype=np.uint32).astype(np.uint16)
    h = h[((h >> 7) & 0xFF) != 0xFF]                      # finite values
    g = reduce_contributions([h])
    w = bf16_to_f32(h)
    assert np.array_equal(g, w + np.float32(0))            # equal values (-0 becomes +0)
    assert not np.signbit(g[h == 0x8000]).any()


def test_start_value_is_plus_zero():
    neg0 = np.array([0x8000], dtype=np.uint16)
    g = reduce_contributions([neg0, neg0, neg0])
    assert g[0] == 0 and not np.signbit(g[0])


def test_scale_applies_once_after_the_sum():
    c = [bf([3.0, -5.0]), bf([1.0, 1.0])]
    assert np.array_equal(reduce_contributions(c, 0.125), np.float32([0.5, -0.5]))


# ---------------------------------------------------------------- AdamW against a library routine

def _torch_adamw_f64(master, grads_f64, steps, hp, record=False):
    p = torch.nn.Parameter(torch.from_numpy(master.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    trace = []
    for t in range(steps):
        p.grad = torch.from_numpy(grads_f64[t])
        opt.step()
        st = opt.state[p]
        trace.append((p.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
                      st["exp_avg_sq"].numpy().copy()))
    return trace if record else trace[-1]


def _f32_budget(trace, grads_f64, hp):
    """Per-element float32 rounding budget of the oracle against an exact-arithmetic run.

    Every float32 operation is within 2^-24 relative of its exact result, and the constants are
    rounded once.  The first moment can cancel, so its budget scales with the moving average of
    |g| rather than with |m|; the weight's budget collects two roundings of the weight per step and
    the update term's own error, including what the moment errors do to it."""
    b1, b2, lr, eps = hp["beta1"], hp["beta2"], hp["lr"], hp["eps"]
    mabs = np.zeros_like(grads_f64[0])
    tol_th = np.zeros_like(grads_f64[0])
    for t, (th, m, v) in enumerate(trace, start=1):
        g = grads_f64[t - 1]
        mabs = b1 * mabs + (1 - b1) * np.abs(g)
        tol_m = 4 * t * U24 * mabs
        tol_v = 4 * t * U24 * v
        bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
        den = np.sqrt(v / bc2) + eps
        ratio = np.abs(m / bc1) / den
        tol_th = tol_th + 3 * U24 * np.abs(th) + lr * (
            12 * U24 * ratio + tol_m / (bc1 * den) + ratio * 4 * t * U24)
    return tol_th, tol_m, tol_v


@pytest.mark.parametrize("gstd", [1e-2, 1e-3, 1e-6])
@pytest.mark.parametrize("wd", [0.01, 0.0, 0.1])
def test_adamw_multi_step_against_library(gstd, wd):
    hp = dict(HP, weight_decay=wd)
    rng = np.random.default_rng(11)
    n, steps, F = 20000, 6, 4
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    master, m, v = master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    grads = []
    for t in range(1, steps + 1):
        contribs = [bf(rng.standard_normal(n) * gstd) for _ in range(F)]
        g = reduce_contributions(contribs)
        grads.append(g.astype(np.float64))
        c = hyper_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], wd, t)
        master, m, v = adamw_update(master, m, v, g, c, np.ones(n, bool), np.ones(n, bool))
    trace = _torch_adamw_f64(master0, grads, steps, hp, record=True)
    th64, m64, v64 = trace[-1]
    tol_th, tol_m, tol_v = _f32_budget(trace, grads, hp)
    assert np.all(np.abs(master - th64) <= tol_th)
    assert np.all(np.abs(m - m64) <= tol_m)
    assert np.all(np.abs(v - v64) <= tol_v)
    # the float64 shadow of the oracle module agrees with the library as well
    th_s, m_s, v_s = master0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, steps + 1):
        th_s, m_s, v_s = adamw_update_f64(th_s, m_s, v_s, grads[t - 1], hp, t, np.ones(n, bool))
    assert np.allclose(th_s, th64, rtol=1e-12, atol=1e-15)


def test_library_pin_detects_planted_mistakes():
    """Each plausible slip in the update (here applied to a copy of the constants) moves the result
    outside the tolerance used above, so the library pin can catch it."""
    rng = np.random.default_rng(12)
    n = 5000
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = bf16_to_f32(bf(rng.standard_normal(n) * 1e-2))
    trace = _torch_adamw_f64(master0, [g.astype(np.float64)], 1, HP, record=True)
    th64 = trace[-1][0]
    tol = _f32_budget(trace, [g.astype(np.float64)], HP)[0]
    ones = np.ones(n, bool)
    good = hyper_constants(**HP, step=1)
    mistakes = [dict(good, bc1=np.float32(1.0)),                 # no first-moment bias correction
                dict(good, bc2=np.float32(1.0)),                 # no second-moment bias correction
                dict(good, dec=np.float32(1.0)),                 # decay dropped
                dict(good, lr=np.float32(-HP["lr"])),            # sign of the step
                dict(good, b1=good["b2"], b2=good["b1"])]        # betas swapped
    th, _, _ = adamw_update(master0, np.zeros(n, np.float32), np.zeros(n, np.float32), g, good, ones, ones)
    assert np.all(np.abs(th - th64) <= tol)
    for bad in mistakes:
        th, _, _ = adamw_update(master0, np.full(n, 1e-3, np.float32), np.full(n, 1e-6, np.float32),
                                g, bad, ones, ones)
        th_ref, _, _ = adamw_update(master0, np.full(n, 1e-3, np.float32), np.full(n, 1e-6, np.float32),
                                    g, good, ones, ones)
        assert np.any(np.abs(th - th_ref) > tol)


# ---------------------------------------------------------------- closed forms

def test_first_step_moves_by_lr_times_sign():
    rng = np.random.default_rng(13)
    n = 100000
    master0 = rng.uniform(-0.05, 0.05, n).astype(np.float32)
    g = bf16_to_f32(bf(rng.standard_normal(n) * 1e-2))
    g[::997] = 0.0
    c = hyper_constants(**HP, step=1)
    ones = np.ones(n, bool)
    th, m, v = adamw_update(master0, np.zeros(n, np.float32), np.zeros(n, np.float32), g, c, ones, ones)
    nz = g != 0
    expect = master0.astype(np.float64) * (1 - HP["lr"] * HP["weight_decay"]) - HP["lr"] * np.sign(g)
    # |g| ~ 1e-2 >> eps: relative deviation of the move ~ eps/|g| plus float32 rounding
    dev = np.abs(th.astype(np.float64) - expect)
    bound = HP["lr"] * (HP["eps"] / np.maximum(np.abs(g), 1e-30) + 16 * U24) + 4 * U24 * np.abs(master0)
    assert np.all(dev[nz] <= bound[nz])
    # g == 0 exactly: the weight is only decayed, bit for bit, and both moments stay zero
    z = ~nz
    assert z.any()
    assert np.array_equal(th[z], master0[z] * np.float32(1 - HP["lr"] * HP["weight_decay"]))
    assert not m[z].any() and not v[z].any()


def test_zero_gradient_only_decays_moments():
    rng = np.random.default_rng(14)
    n = 10000
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = (rng.random(n) * 1e-6).astype(np.float32)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    c = hyper_constants(**HP, step=7)
    ones = np.ones(n, bool)
    th, m, v = adamw_update(th0, m0, v0, np.zeros(n, np.float32), c, ~ones, ones)
    assert np.array_equal(m, m0 * np.float32(HP["beta1"]))
    assert np.array_equal(v, v0 * np.float32(HP["beta2"]))
    # without the decay flag and with zero moments the weight does not move at all
    th, _, _ = adamw_update(th0, np.zeros(n, np.float32), np.zeros(n, np.float32),
                            np.zeros(n, np.float32), c, ~ones, ones)
    assert np.array_equal(th, th0)


def test_padding_keeps_state_and_outputs_zero():
    rng = np.random.default_rng(15)
    n = 64
    flags = np.array([layout.WEIGHT_DECAY] * 40 + [layout.WEIGHT_DECAY | layout.PADDING] * 24)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = (rng.random(n) * 1e-6).astype(np.float32)
    contribs = [bf(rng.standard_normal(n) * 1e-2) for _ in range(3)]
    contribs[1][40:] = 0x7FC0                                   # NaN gradients in the padding
    th, m, v, out = shard_step(th0, m0, v0, contribs, flags, HP, 3)
    pad = slice(40, None)
    assert th[pad].tobytes() == th0[pad].tobytes()
    assert m[pad].tobytes() == m0[pad].tobytes() and v[pad].tobytes() == v0[pad].tobytes()
    assert not out[pad].any()
    assert np.isfinite(th[:40]).all()
    assert np.array_equal(out[:40], f32_to_bf16_rne(th[:40]))


def test_constants_follow_the_step_counter():
    c1 = hyper_constants(**HP, step=1)
    assert c1["bc1"] == np.float32(0.1) and c1["bc2"] == np.float32(1 - 0.999)
    c10 = hyper_constants(**HP, step=10)
    assert c10["bc1"] == np.float32(1 - 0.9 ** 10)
    with pytest.raises(ValueError):
        hyper_constants(**HP, step=0)
