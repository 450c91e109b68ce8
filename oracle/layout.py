"""Flat layout and floor-rule shard boundaries (oracle; test infrastructure only).

Source: "FSDP: Fully Sharded Data Parallel Training at Scale", the passage on sharding a linear
layer. A unit's parameters are viewed as one 1-D tensor of length P; with N ranks, rank k owns the
contiguous elements floor(kP/N) through floor((k+1)P/N) - 1, and the gradient shard and the Adam
m / v shards cover exactly the same positions, so the optimizer update of a slice is local.

Everything here is plain Python integers (arbitrary precision), so k*P never overflows.

Readings taken where the pages are silent:
* Several tensors are flattened in the order given, each optionally padded up to a multiple of
  ``pad_multiple`` elements; padding elements are part of the flat vector (they occupy flat
  positions and are sharded like any other element) but are never updated.
* A per-tensor weight-decay flag travels with each segment.
* P < N is legal: some ranks then own an empty slice.
"""

import numpy as np

WEIGHT_DECAY = 1  # segment flag: decoupled weight decay applies to these elements
PADDING = 2       # segment flag: padding elements (never updated, bf16 output +0)


def padded_size(size, pad_multiple):
    """Smallest multiple of ``pad_multiple`` that is >= ``size``."""
    if pad_multiple < 1:
        raise ValueError("pad_multiple must be >= 1")
    if size < 0:
        raise ValueError("tensor sizes must be >= 0")
    return -(-size // pad_multiple) * pad_multiple


def flatten_offsets(sizes, pad_multiple=1):
    """Start offset of every tensor in the flat vector, and the flat length P.

    Tensor i occupies flat positions [offsets[i], offsets[i] + sizes[i]) for its real elements,
    followed by padded_size(sizes[i]) - sizes[i] padding elements.
    """
    offsets = []
    pos = 0
    for s in sizes:
        offsets.append(pos)
        pos += padded_size(int(s), pad_multiple)
    return offsets, pos


def shard_bounds(P, N, k):
    """[lo, hi) of rank k: lo = floor(kP/N), hi = floor((k+1)P/N)."""
    if N < 1:
        raise ValueError("world size must be >= 1")
    if not 0 <= k < N:
        raise ValueError("rank must satisfy 0 <= k < N")
    if P < 0:
        raise ValueError("P must be >= 0")
    return (k * P) // N, ((k + 1) * P) // N


def segments(sizes, pad_multiple, wd_mask, N, k):
    """Ordered pieces of rank k's slice, one per (tensor, real-or-padding) run.

    Returns (lo, hi, segs) where every entry of segs is a dict with
      shard_begin   -- first element, counted from lo
      length        -- number of elements (>= 1)
      tensor_id     -- index of the tensor the run belongs to
      tensor_offset -- position of shard_begin inside that tensor's padded extent
      flags         -- WEIGHT_DECAY and/or PADDING
    The runs tile [0, hi - lo) in order with no gap and no overlap.
    """
    offsets, P = flatten_offsets(sizes, pad_multiple)
    lo, hi = shard_bounds(P, N, k)
    segs = []
    for i, s in enumerate(sizes):
        s = int(s)
        wd = WEIGHT_DECAY if (wd_mask is None or bool(wd_mask[i])) else 0
        base = offsets[i]
        for a, b, flags in ((base, base + s, wd),
                            (base + s, base + padded_size(s, pad_multiple), wd | PADDING)):
            x, y = max(a, lo), min(b, hi)
            if x < y:
                segs.append(dict(shard_begin=x - lo, length=y - x, tensor_id=i,
                                 tensor_offset=x - base, flags=flags))
    return lo, hi, segs


def element_flags(segs, n):
    """Per-element flags of a slice of length n, expanded from its segments (lists of ints)."""
    flags = [None] * n
    for sg in segs:
        for j in range(sg["shard_begin"], sg["shard_begin"] + sg["length"]):
            flags[j] = sg["flags"]
    return flags
