"""Shared helpers of the GPU parity tests: guarded device buffers and comparison bars.

Comparison bars (fp32 state: relative 1e-5; bf16 params: at most 1 ulp, measured as the distance
of the two bit patterns on the ordered-integer line; NaN matches NaN, since the two sides may
produce different NaN payloads).
"""

import numpy as np
import torch

F32_RTOL = 1e-5
BF16_ULP = 1
GUARD = 64                          # elements of guard band on each side of every buffer
SENT32 = np.uint32(0x7FA5A5A5)      # signalling-NaN pattern no kernel writes by itself
SENT16 = np.uint16(0x7FA5)


def say(msg):
    print(msg, flush=True)


class Guarded:
    """A device buffer with sentinel-filled guard bands around the region the call may touch."""

    def __init__(self, host, guard=GUARD, pre=0):
        host = np.ascontiguousarray(host)
        self.dtype = host.dtype
        self.n = host.size
        self.guard = guard
        self.pre = pre                      # elements between the guard and `host` (also guarded)
        total = guard + pre + self.n + guard
        if host.dtype == np.float32:
            fill = np.full(total, SENT32, dtype=np.uint32).view(np.float32)
        else:
            fill = np.full(total, SENT16, dtype=np.uint16).view(host.dtype)
        fill[guard + pre: guard + pre + self.n] = host
        tdt = torch.float32 if host.dtype == np.float32 else torch.int16
        raw = fill.view(np.int16) if host.dtype == np.uint16 else fill
        self.full = torch.from_numpy(raw.copy()).to("cuda")
        self.sentinel = fill.copy()
        assert self.full.dtype == tdt

    def window(self, start_elem=None):
        """View starting `pre` elements before the data (the guarded prefix) or at `start_elem`."""
        s = self.guard if start_elem is None else start_elem
        return self.full[s:]

    def data(self):
        return self.full[self.guard + self.pre: self.guard + self.pre + self.n]

    def host(self):
        h = self.full.cpu().numpy()
        return h.view(np.uint16) if self.dtype == np.uint16 else h

    def data_host(self):
        return self.host()[self.guard + self.pre: self.guard + self.pre + self.n]

    def assert_guards(self, what):
        h = self.host()
        a, b = self.guard + self.pre, self.guard + self.pre + self.n
        ref = self.sentinel.view(np.uint16) if self.dtype == np.uint16 else self.sentinel
        bad_lo = np.flatnonzero(h[:a].view(np.uint8) != ref[:a].view(np.uint8))
        bad_hi = np.flatnonzero(h[b:].view(np.uint8) != ref[b:].view(np.uint8))
        assert bad_lo.size == 0 and bad_hi.size == 0, f"{what}: guard band written"


def ordered16(h):
    """bf16 bit patterns mapped to integers in value order (+0 and -0 both map to 0)."""
    h = h.astype(np.int32)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def assert_f32(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    nan = np.isnan(got) & np.isnan(want)
    same = got.view(np.uint32) == want.view(np.uint32)
    with np.errstate(invalid="ignore"):   # inf - inf: those elements are settled by `same`
        close = np.abs(got.astype(np.float64) - want) <= F32_RTOL * np.abs(want.astype(np.float64))
    ok = nan | same | close
    if not ok.all():
        i = np.flatnonzero(~ok)[:5]
        raise AssertionError(f"{what}: {(~ok).sum()} mismatches, e.g. at {i}: "
                             f"got {got[i]} want {want[i]}")


def assert_bf16(got, want, what):
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    isnan = lambda h: ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    nan = isnan(got) & isnan(want)
    dist = np.abs(ordered16(got) - ordered16(want))
    ok = nan | (dist <= BF16_ULP)
    if not ok.all():
        i = np.flatnonzero(~ok)[:5]
        raise AssertionError(f"{what}: {(~ok).sum()} mismatches, e.g. at {i}: "
                             f"got {[hex(x) for x in got[i]]} want {[hex(x) for x in want[i]]}")


def bit_equal(got, want):
    """Equal bit patterns, NaN matching any NaN."""
    got = np.asarray(got)
    want = np.asarray(want)
    if got.dtype == np.float32:
        nan = np.isnan(got) & np.isnan(want)
        return bool(np.all(nan | (got.view(np.uint32) == want.view(np.uint32))))
    isnan = lambda h: ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    return bool(np.all((isnan(got) & isnan(want)) | (got == want)))


def to_dev16(h):
    return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).to("cuda")
