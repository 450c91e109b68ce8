"""Bytes of training state per parameter and per rank (oracle; test infrastructure only).

Sources (page titles as published):
* "FSDP: Fully Sharded Data Parallel Training at Scale"
  - memory breakdown: float32 training keeps 4 B of parameter, 4 B of gradient and 8 B of Adam
    moments per parameter (16P bytes); the common mixed-precision accounting is 2 (bf16 param) +
    2 (bf16 grad) + 4 (fp32 master) + 8 (fp32 moments), again 16P.
  - FULL_SHARD memory: each of the N ranks keeps 16P/N at rest; while one of M units is gathered
    the peak adds that unit's full float32 parameters, 4P/M.
  - SHARD_GRAD_OP: gradients and optimizer state (12P in float32) are divided by N, parameters are
    not, so the saving is 12P(N-1)/N; FULL_SHARD saves 16P(N-1)/N.
* "Distributed Deep Learning & Model Sharding", "The constraint is rarely FLOPs": about 16 B per
  parameter with bf16 weights and grads and ~12 B of fp32 master plus first and second moments.

All results are exact integers (bytes) or Fractions; callers convert units.
"""

from fractions import Fraction

# Per-parameter byte costs of each component.
MIXED = dict(param=2, grad=2, master=4, moments=8)   # bf16 param/grad, fp32 master and m, v
FP32 = dict(param=4, grad=4, master=0, moments=8)    # float32 training, no separate master


def bytes_per_param(scheme=MIXED):
    return sum(scheme.values())


def adam_state_bytes(P, scheme=MIXED):
    """Optimizer-owned bytes: fp32 master (if any) plus the two fp32 moments."""
    return P * (scheme["master"] + scheme["moments"])


def model_state_bytes(P, scheme=MIXED):
    return P * bytes_per_param(scheme)


def full_shard_per_rank(P, N, scheme=MIXED):
    """Steady-state bytes per rank under full sharding (every component divided by N)."""
    return Fraction(model_state_bytes(P, scheme), N)


def full_shard_peak(P, N, M, scheme=FP32):
    """Full-shard steady state plus one gathered unit of P/M parameters at param precision."""
    return full_shard_per_rank(P, N, scheme) + Fraction(P * scheme["param"], M)


def shard_grad_op_saving(P, N, scheme=FP32):
    """Bytes per rank saved by sharding only gradients and optimizer state."""
    sharded = scheme["grad"] + scheme["master"] + scheme["moments"]
    return Fraction(P * sharded * (N - 1), N)


def full_shard_saving(P, N, scheme=FP32):
    """Bytes per rank saved by sharding every component."""
    return Fraction(model_state_bytes(P, scheme) * (N - 1), N)


def shard_state_bytes(n):
    """Bytes at rest of one n-element shard in the mixed-precision layout (2+2+4+8 per element)."""
    return n * bytes_per_param(MIXED)
