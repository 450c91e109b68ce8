"""Pins for the oracle's reshard: identities and brute force, nothing that re-types its code.

* Round trips N -> N' -> N return the original shards exactly (same padding).
* Whatever the world size, the concatenated shards are the same flat vector (the full state dict
  of the checkpointing passage in "FSDP: Fully Sharded Data Parallel Training at Scale").
* Per-element brute force on small cases: element j of tensor i sits at padded offset o_i + j in
  both layouts, and destination padding is zero.
"""

import random

import numpy as np
import pytest

from oracle import layout, reshard


def _rand_case(rng):
    T = rng.randint(1, 7)
    sizes = [rng.randint(0, 40) for _ in range(T)]
    return sizes, rng.choice([1, 2, 8, 16]), rng.choice([1, 2, 8, 16])


def test_round_trip_same_padding():
    rng = random.Random(1)
    for trial in range(200):
        sizes, pad, _ = _rand_case(rng)
        offs, P = layout.flatten_offsets(sizes, pad)
        flat = np.zeros(P, dtype=np.float32)               # padding is zero after a reshard
        for o, s in zip(offs, sizes):
            flat[o:o + s] = np.arange(o, o + s) + 0.5
        for N in (1, 2, 3, 8):
            shards = reshard.shard(flat, sizes, pad, N)
            for N2 in (1, 4, 5, 16):
                there = reshard.reshard(shards, sizes, pad, pad, N2)
                back = reshard.reshard(there, sizes, pad, pad, N)
                assert all(np.array_equal(a, b) for a, b in zip(back, shards))
                assert np.array_equal(np.concatenate(there), flat)


def test_brute_force_padding_change():
    rng = random.Random(2)
    for trial in range(200):
        sizes, pad_a, pad_b = _rand_case(rng)
        offs_a, P_a = layout.flatten_offsets(sizes, pad_a)
        offs_b, P_b = layout.flatten_offsets(sizes, pad_b)
        flat_a = np.full(P_a, -7.0, dtype=np.float32)               # padding holds junk
        for i, (o, s) in enumerate(zip(offs_a, sizes)):
            flat_a[o:o + s] = 1000 * i + np.arange(s)
        N_a, N_b = rng.randint(1, 9), rng.randint(1, 9)
        out = reshard.reshard(reshard.shard(flat_a, sizes, pad_a, N_a), sizes, pad_a, pad_b, N_b)
        flat_b = np.concatenate(out) if out else np.zeros(0, np.float32)
        assert flat_b.size == P_b
        expect = np.zeros(P_b, dtype=np.float32)
        for i, (o, s) in enumerate(zip(offs_b, sizes)):
            for j in range(s):
                expect[o + j] = 1000 * i + j
        assert np.array_equal(flat_b, expect)
        for k, part in enumerate(out):
            lo, hi = layout.shard_bounds(P_b, N_b, k)
            assert part.size == hi - lo


@pytest.mark.parametrize("dtype", [np.float32, np.uint16, np.float64])
def test_dtype_kept(dtype):
    sizes = [5, 3]
    out = reshard.reshard(reshard.shard(np.arange(8).astype(dtype), sizes, 1, 2), sizes, 1, 4, 3)
    assert all(o.dtype == dtype for o in out)
    assert np.concatenate(out).tolist() == [0, 1, 2, 3, 4, 0, 0, 0, 5, 6, 7, 0]
