"""Pins for the oracle's flat layout and floor-rule shards.

The rule itself comes from "FSDP: Fully Sharded Data Parallel Training at Scale" (passage on
sharding a linear layer): rank k owns floor(kP/N) .. floor((k+1)P/N)-1.  The pins below check it
against things other than the formula: the page's own statements for GPU 0 and GPU 1, an
independent closed form for the owner of each element, partition invariants, and per-element
brute force for the segment table.
"""

import itertools
import random

import numpy as np

import pytest

from oracle import layout


def owner_of(i, P, N):
    """Owner of flat element i derived by hand from the floor rule: floor(kP/N) <= i iff
    kP < (i+1)N, and i < floor((k+1)P/N) iff (i+1)N <= (k+1)P; so k = ceil((i+1)N/P) - 1."""
    return -(-((i + 1) * N) // P) - 1


@pytest.mark.parametrize("N", range(1, 18))
def test_partition_brute_force(N):
    for P in range(0, 301):
        bounds = [layout.shard_bounds(P, N, k) for k in range(N)]
        assert bounds[0][0] == 0 and bounds[-1][1] == P
        for k in range(N - 1):
            assert bounds[k][1] == bounds[k + 1][0]          # no gap, no overlap
        sizes = [hi - lo for lo, hi in bounds]
        assert sum(sizes) == P
        assert set(sizes) <= {P // N, -(-P // N)}             # balanced to within one element
        for k, (lo, hi) in enumerate(bounds):
            for i in range(lo, hi):
                assert owner_of(i, P, N) == k


def test_page_statements_for_gpu0_and_gpu1():
    # GPU 0 holds 0 .. floor(P/N)-1 and GPU 1 holds floor(P/N) .. floor(2P/N)-1.
    for P, N in [(1000003, 8), (218112000, 8), (7, 3), (100, 7)]:
        assert layout.shard_bounds(P, N, 0) == (0, P // N)
        assert layout.shard_bounds(P, N, 1) == (P // N, (2 * P) // N)


def test_worked_values():
    # P = 1,000,003 over 8 ranks: k*P/8 = 125000.375 k, floored.
    P, N = 1000003, 8
    edges = [layout.shard_bounds(P, N, k)[0] for k in range(N)] + [P]
    assert edges == [0, 125000, 250000, 375001, 500001, 625001, 750002, 875002, 1000003]
    # P < N: five of eight ranks are empty.
    edges = [layout.shard_bounds(3, 8, k)[0] for k in range(8)] + [3]
    assert edges == [0, 0, 0, 1, 1, 1, 2, 2, 3]


def test_large_values_are_exact():
    # k*P exceeds 2**63 here; Python integers keep it exact.
    P, N = (1 << 62) + 12345, 64
    for k in (0, 1, 31, 63):
        lo, hi = layout.shard_bounds(P, N, k)
        assert lo * N <= k * P < (lo + 1) * N
        assert hi * N <= (k + 1) * P < (hi + 1) * N


def test_padding_and_offsets():
    offs, P = layout.flatten_offsets([5, 16, 1, 0, 17], 16)
    assert offs == [0, 16, 32, 48, 48] and P == 80
    offs, P = layout.flatten_offsets([5, 16, 1], 1)
    assert offs == [0, 5, 21] and P == 22


def _brute_segments(sizes, pad, wd, N, k):
    """Per-element (tensor, offset, flags) of rank k's slice by walking every flat position."""
    flat = []
    for t, s in enumerate(sizes):
        for j in range(layout.padded_size(s, pad)):
            f = (layout.WEIGHT_DECAY if (wd is None or wd[t]) else 0)
            if j >= s:
                f |= layout.PADDING
            flat.append((t, j, f))
    lo, hi = layout.shard_bounds(len(flat), N, k)
    return flat[lo:hi]


def test_segments_brute_force():
    rng = random.Random(7)
    for trial in range(300):
        T = rng.randint(1, 6)
        sizes = [rng.randint(0, 23) for _ in range(T)]
        pad = rng.choice([1, 1, 4, 16])
        wd = [rng.random() < 0.5 for _ in range(T)] if rng.random() < 0.7 else None
        N = rng.randint(1, 9)
        cover = {}
        for k in range(N):
            lo, hi, segs = layout.segments(sizes, pad, wd, N, k)
            expect = _brute_segments(sizes, pad, wd, N, k)
            got = []
            pos = 0
            for sg in segs:
                assert sg["shard_begin"] == pos and sg["length"] >= 1
                pos += sg["length"]
                for j in range(sg["length"]):
                    got.append((sg["tensor_id"], sg["tensor_offset"] + j, sg["flags"]))
            assert pos == hi - lo
            assert got == expect
            for idx, e in enumerate(got):
                assert (e[0], e[1]) not in cover
                cover[(e[0], e[1])] = k
        # The union over ranks covers every (tensor, padded position) exactly once.
        total = sum(layout.padded_size(s, pad) for s in sizes)
        assert len(cover) == total


def test_segment_runs_merge_only_at_edges():
    # Adjacent segments always differ in tensor or in padding status.
    lo, hi, segs = layout.segments([10, 3, 7], 8, [True, False, True], 3, 1)
    for a, b in zip(segs, segs[1:]):
        assert (a["tensor_id"], a["flags"] & layout.PADDING) != (b["tensor_id"], b["flags"] & layout.PADDING)


@pytest.mark.parametrize("bad", [dict(P=5, N=0, k=0), dict(P=5, N=2, k=2), dict(P=5, N=2, k=-1),
                                 dict(P=-1, N=2, k=0)])
def test_rejects_bad_arguments(bad):
    with pytest.raises(ValueError):
        layout.shard_bounds(bad["P"], bad["N"], bad["k"])


def test_element_flags_expand():
    lo, hi, segs = layout.segments([3, 2], 4, [False, True], 2, 0)
    flags = layout.element_flags(segs, hi - lo)
    assert flags == [0, 0, 0, layout.PADDING]
    lo, hi, segs = layout.segments([3, 2], 4, [False, True], 2, 1)
    W, Pd = layout.WEIGHT_DECAY, layout.PADDING
    assert layout.element_flags(segs, hi - lo) == [W, W, W | Pd, W | Pd]


def test_owner_closed_form_is_not_the_formula_itself():
    # Guard against a degenerate pin: the closed form must disagree with a wrong rule, e.g. ceil.
    P, N = 10, 4
    wrong = [(-(-k * P // N), -(-(k + 1) * P // N)) for k in range(N)]
    right = [layout.shard_bounds(P, N, k) for k in range(N)]
    assert wrong != right
    for k, (lo, hi) in enumerate(right):
        assert all(owner_of(i, P, N) == k for i in range(lo, hi))
    assert list(itertools.chain.from_iterable(range(lo, hi) for lo, hi in right)) == list(range(P))
