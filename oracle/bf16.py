"""bfloat16 <-> float32 on bit patterns (oracle; test infrastructure only).

Source: "FSDP: Fully Sharded Data Parallel Training at Scale", mixed-precision passage: bfloat16
has the same 8-bit exponent as float32 and a 7-bit mantissa (float32 has 23), so a bf16 value is
the top 16 bits of a float32.

Readings taken where the pages are silent:
* float32 -> bf16 rounds to nearest, ties to even (IEEE 754 default rounding), on the bit
  pattern: add 0x7FFF plus the lowest kept bit, then keep the high half.  Values that round past
  the largest finite bf16 become +-Inf, as IEEE rounding prescribes.
* NaN stays NaN with its sign and its top payload bits, and is made quiet (bit 6 of the bf16
  mantissa set).
* bf16 -> float32 is exact: shift the 16 bits into the high half.
bf16 values are held as numpy uint16 arrays.
"""

import numpy as np


def bf16_to_f32(h):
    """Exact widening of bf16 bit patterns (uint16 array) to float32."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x):
    """Round float32 values to bf16 bit patterns (uint16), nearest-even; NaN made quiet."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)  # widen so the rounding add cannot wrap
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint32)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet_nan = ((u >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint32)
    out = np.where(is_nan, quiet_nan, rounded)
    return (out & np.uint32(0xFFFF)).astype(np.uint16)
