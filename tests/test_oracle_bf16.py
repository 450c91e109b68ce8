"""Pins for the oracle's bf16 conversion.

bfloat16 is float32's sign and 8-bit exponent with a 7-bit mantissa ("FSDP: Fully Sharded Data
Parallel Training at Scale", mixed-precision passage).  The rounding rule (nearest, ties to even)
is IEEE 754's default.  Pins: an independent nearest-value search in exact rational arithmetic, a
library routine (PyTorch's CPU float32 -> bfloat16 conversion, which rounds to nearest even), and
special values.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle.bf16 import bf16_to_f32, f32_to_bf16_rne


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def _bf16_value(h):
    """Exact value of a finite bf16 bit pattern, decoded by hand from sign/exponent/mantissa."""
    s = -1 if h & 0x8000 else 1
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    if e == 0:
        return s * Fraction(f, 128) * Fraction(2) ** -126
    return s * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)


def _nearest_even(x):
    """Nearest non-negative bf16 pattern to the fraction x >= 0 by searching the neighbours;
    ties go to the even mantissa.  Magnitudes at or beyond the rounding threshold of the largest
    finite value go to infinity."""
    max_fin = _bf16_value(0x7F7F)
    half_ulp_top = Fraction(2) ** (127 - 8)
    a = x
    if a >= max_fin + half_ulp_top:
        return 0x7F80
    # candidate: largest non-negative pattern with value <= a
    lo, hi = 0, 0x7F7F
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if _bf16_value(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    below = lo
    above = below + 1
    db = a - _bf16_value(below)
    da = (_bf16_value(above) - a) if above <= 0x7F7F else (max_fin + 2 * half_ulp_top - a)
    if db < da:
        pick = below
    elif da < db:
        pick = above
    else:
        pick = below if below % 2 == 0 else above
    return pick


def test_exact_values_roundtrip():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(h)
    finite = ~np.isnan(x)
    assert np.array_equal(f32_to_bf16_rne(x[finite]), h[finite])


def test_widening_matches_hand_decoding():
    rng = np.random.default_rng(1)
    for h in list(rng.integers(0, 1 << 16, 400)) + [0, 0x8000, 0x0001, 0x8001, 0x7F7F, 0x0080]:
        h = int(h)
        if (h >> 7) & 0xFF == 0xFF:
            continue
        assert Fraction(float(bf16_to_f32(np.uint16(h)))) == _bf16_value(h)


def test_rounding_against_exact_nearest():
    rng = np.random.default_rng(2)
    bits = list(rng.integers(0, 0x7F800000, 3000, dtype=np.uint32))
    # ties (low half exactly 0x8000) with odd and even kept bit, and their neighbours
    for hi in list(rng.integers(0, 0x7F80, 200)) + [0x0000, 0x0001, 0x3F80, 0x3F81, 0x7F7E, 0x7F7F]:
        for low in (0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF):
            bits.append((int(hi) << 16) | low)
    for b in bits:
        for sgn in (0, 0x80000000):
            x = _f32(int(b) | sgn)
            got = int(f32_to_bf16_rne(np.float32(x)))
            want = _nearest_even(abs(Fraction(float(x)))) | (0x8000 if sgn else 0)
            assert got == want, hex(int(b) | sgn)


def test_against_library_conversion():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    lib = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(x), lib)
    y = (rng.standard_normal(1_000_000) * 1e-2).astype(np.float32)
    lib = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(y), lib)


def test_special_values():
    cases = {
        0x00000000: 0x0000,      # +0
        0x80000000: 0x8000,      # -0 keeps its sign
        0x7F800000: 0x7F80,      # +Inf
        0xFF800000: 0xFF80,      # -Inf
        0x7F7FFFFF: 0x7F80,      # largest finite float32 rounds up to +Inf
        0xFF7FFFFF: 0xFF80,
        0x7F7F7FFF: 0x7F7F,      # just below the tie: stays at the largest finite bf16
        0x7F7F8000: 0x7F80,      # tie with odd kept bit rounds to even = Inf
        0x3F808000: 0x3F80,      # 1 + half a bf16 ulp: tie, kept bit even -> 1.0
        0x3F818000: 0x3F82,      # tie, kept bit odd -> up
        0x00000001: 0x0000,      # smallest float32 denormal rounds to +0
        0x00008000: 0x0000,      # tie at zero stays at zero (even)
        0x00018000: 0x0002,      # tie with odd kept bit goes up
    }
    for b, want in cases.items():
        assert int(f32_to_bf16_rne(_f32(b))) == want, hex(b)


def test_nan_stays_nan_quiet_and_signed():
    for b in (0x7FC00000, 0x7F800001, 0x7FBFFFFF, 0xFFC00001, 0xFF800001, 0x7FFFFFFF):
        h = int(f32_to_bf16_rne(_f32(b)))
        assert (h >> 7) & 0xFF == 0xFF and h & 0x7F != 0          # NaN
        assert h & 0x40                                           # quiet
        assert (h & 0x8000) == ((b >> 16) & 0x8000)               # sign kept
