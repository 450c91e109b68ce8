"""Reduce + AdamW + bf16 unflatten on one rank's slice (oracle; test infrastructure only).

Sources (page titles as published):
* "FSDP: Fully Sharded Data Parallel Training at Scale"
  - communication pattern of one FSDP unit: after backward, a reduce-scatter sums the ranks'
    gradients and hands rank k only the part that matches its parameter slice; the optimizer
    step then runs on each rank with its own gradient, parameter and optimizer-state slices and
    needs no communication; before the next forward an all-gather rebuilds the full parameters
    from every rank's slice.
  - memory breakdown: Adam keeps a first moment (exponential moving average of the gradient) and a
    second moment (exponential moving average of the squared gradient), both in float32; the
    mixed-precision accounting is bf16 params + bf16 grads + fp32 master params + fp32 moments.
  - mixed precision: the gradient reduction runs in float32 (reduce_dtype) while parameters and
    all-gather buffers are bf16.
* "Distributed Deep Learning & Model Sharding", section "The constraint is rarely FLOPs": bf16
  weights and gradients plus fp32 master weights and first and second moments.

The pages name Adam / AdamW but do not print its equations.  Reading used (Kingma & Ba's
bias-corrected Adam with Loshchilov & Hutter's decoupled weight decay, the decay scaled by the
learning rate), per real element, every operation an IEEE float32 operation rounded on its own:

    g   = ((+0 + G_0) + G_1) + ... + G_{F-1}      contributions widened from bf16, rank order
    g   = g * grad_scale
    m   = b1*m + c1*g                            c1 = f32(1 - beta1)
    v   = b2*v + c2*(g*g)                        c2 = f32(1 - beta2)
    mh  = m / bc1                                bc1 = f32(1 - beta1**t)
    vh  = v / bc2                                bc2 = f32(1 - beta2**t)
    den = sqrt(vh) + eps
    th  = th * dec          (weight-decay flag)  dec = f32(1 - lr*weight_decay)
    th  = th - lr*(mh/den)
    out = bf16_rne(th)

Scalar constants are formed in float64 from the float64 hyperparameters and rounded to float32
once.  The step counter t is 1-based.  Padding elements keep master, m and v bit for bit and
produce a +0 bf16 output; their gradient values are ignored (they may be NaN).
"""

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16_rne
from .layout import PADDING, WEIGHT_DECAY

F32 = np.float32


def hyper_constants(lr, beta1, beta2, eps, weight_decay, step, grad_scale=1.0):
    """float32 constants of step ``step`` (1-based), each from one float64 expression."""
    if step < 1:
        raise ValueError("the step counter is 1-based")
    return dict(
        b1=F32(beta1), b2=F32(beta2),
        c1=F32(1.0 - beta1), c2=F32(1.0 - beta2),
        bc1=F32(1.0 - beta1 ** step), bc2=F32(1.0 - beta2 ** step),
        eps=F32(eps), lr=F32(lr),
        dec=F32(1.0 - lr * weight_decay),
        scale=F32(grad_scale),
    )


def reduce_contributions(contribs, grad_scale=1.0):
    """fp32 sum of bf16 contributions in rank order 0..F-1, starting from +0, then scaled.

    ``contribs`` is a sequence of F uint16 arrays of equal length (bf16 bit patterns).
    """
    if len(contribs) == 0:
        raise ValueError("at least one contribution is needed")
    g = np.zeros(np.asarray(contribs[0]).shape, dtype=F32)
    for c in contribs:
        g = g + bf16_to_f32(c)
    return g * F32(grad_scale)


def adamw_update(master, m, v, g, consts, wd_on, real):
    """One AdamW update in float32; returns new (master, m, v) arrays, inputs untouched.

    wd_on, real: boolean arrays (decay applies / element is not padding).
    """
    c = consts
    m1 = c["b1"] * m + c["c1"] * g
    v1 = c["b2"] * v + c["c2"] * (g * g)
    mh = m1 / c["bc1"]
    vh = v1 / c["bc2"]
    den = np.sqrt(vh) + c["eps"]
    th = np.where(wd_on, master * c["dec"], master)
    th = th - c["lr"] * (mh / den)
    # Padding keeps its state bit for bit.
    return (np.where(real, th, master).astype(F32),
            np.where(real, m1, m).astype(F32),
            np.where(real, v1, v).astype(F32))


def unflatten_bf16(master, real):
    """bf16 bits of the slice as the all-gather serves them: bf16_rne(master), +0 for padding."""
    out = f32_to_bf16_rne(master)
    return np.where(real, out, np.uint16(0)).astype(np.uint16)


def flags_to_masks(flags):
    """Expand per-element segment flags (int array) into (wd_on, real) boolean arrays."""
    flags = np.asarray(flags)
    return (flags & WEIGHT_DECAY) != 0, (flags & PADDING) == 0


def shard_step(master, m, v, contribs, flags, hp, step):
    """One full step on a slice: reduce, AdamW, bf16 output.  Returns (master, m, v, out_bf16).

    ``hp`` holds lr, beta1, beta2, eps, weight_decay and optionally grad_scale (floats).
    ``flags`` is the per-element segment flag array of the slice.
    """
    consts = hyper_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                             hp["weight_decay"], step, hp.get("grad_scale", 1.0))
    wd_on, real = flags_to_masks(flags)
    g = reduce_contributions(contribs, hp.get("grad_scale", 1.0))
    master, m, v = adamw_update(master, m, v, g, consts, wd_on, real)
    return master, m, v, unflatten_bf16(master, real)


def accumulate_fp32(acc, contribs, scale=1.0):
    """fp32 gradient-shard accumulation across micro-batches: acc + scale * (rank-order sum).

    "FSDP: Fully Sharded Data Parallel Training at Scale", mixed-precision passage (gradients
    accumulate in float32 so small values are not lost) and the note that gradient accumulation
    over micro-batches suppresses synchronisation until the last one.  One float32 rounding for
    the reduction (as reduce_contributions), one for the scale, one for the addition.
    """
    return (np.asarray(acc, np.float32) + reduce_contributions(contribs, scale)).astype(F32)


def shard_step_f32grad(master, m, v, grad, flags, hp, step):
    """One step from an fp32 gradient shard (accumulated over micro-batches): g = grad * scale,
    then the same AdamW and bf16 output as shard_step."""
    consts = hyper_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                             hp["weight_decay"], step, hp.get("grad_scale", 1.0))
    wd_on, real = flags_to_masks(flags)
    g = np.asarray(grad, np.float32) * consts["scale"]
    master, m, v = adamw_update(master, m, v, g, consts, wd_on, real)
    return master, m, v, unflatten_bf16(master, real)


def adamw_update_f64(master, m, v, g, hp, step, wd_on):
    """Diagnostic float64 shadow of the same recurrence (not a pass/fail reference)."""
    master = np.asarray(master, dtype=np.float64)
    m = hp["beta1"] * np.asarray(m, np.float64) + (1.0 - hp["beta1"]) * g
    v = hp["beta2"] * np.asarray(v, np.float64) + (1.0 - hp["beta2"]) * g * g
    mh = m / (1.0 - hp["beta1"] ** step)
    vh = v / (1.0 - hp["beta2"] ** step)
    th = np.where(wd_on, master * (1.0 - hp["lr"] * hp["weight_decay"]), master)
    th = th - hp["lr"] * mh / (np.sqrt(vh) + hp["eps"])
    return th, m, v
