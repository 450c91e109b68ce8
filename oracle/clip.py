"""Global gradient-norm clipping of a sharded gradient (oracle; test infrastructure only).

Source: "FSDP: Fully Sharded Data Parallel Training at Scale", passage on gradient clipping: with
sharded gradients each rank sees only its slice, so a norm computed from one rank's slice
underestimates the norm of the whole gradient; the sharded clip has to combine the ranks' parts
into the true global norm before it scales anything.

Reading used (the pages name the operation but print no formula):
* the clipped quantity is the reduced gradient g (the rank-order fp32 sum of the contributions,
  times grad_scale); padding elements do not count;
* the global squared norm is the sum over ranks of each rank's sum of g_i^2; each g_i is float32,
  so g_i^2 is exact in float64 and the oracle sums the squares exactly (math.fsum, one rounding);
* the clip coefficient follows the common convention max_norm / (norm + 1e-6), capped at 1,
  formed in float64; the step then uses grad_scale * coefficient, rounded to float32 once, in
  place of grad_scale.
"""

import math

import numpy as np

from .step import reduce_contributions

CLIP_EPS = 1e-6


def sumsq_exact(g_f32, real=None):
    """Exactly rounded float64 sum of squares of the float32 values g (real elements only)."""
    g = np.asarray(g_f32, dtype=np.float32)
    if real is not None:
        g = g[np.asarray(real, dtype=bool)]
    sq = g.astype(np.float64) ** 2          # exact: a float32 square needs at most 48 bits
    return math.fsum(sq.tolist())


def grad_sumsq(contribs, real, grad_scale=1.0):
    """Sum of squares of one slice's reduced gradient (the rank's share of the global norm)."""
    return sumsq_exact(reduce_contributions(contribs, grad_scale), real)


def clip_coefficient(global_sumsq, max_norm):
    """min(1, max_norm / (sqrt(global_sumsq) + 1e-6)) in float64."""
    coef = max_norm / (math.sqrt(global_sumsq) + CLIP_EPS)
    return min(1.0, coef)


def clipped_scale(global_sumsq, max_norm, grad_scale=1.0):
    """float32 scale the step applies to the summed contributions when clipping is on."""
    return np.float32(grad_scale * clip_coefficient(global_sumsq, max_norm))
