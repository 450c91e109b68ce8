"""Resharding a flat, floor-rule-sharded vector to another world size (oracle; test only).

Source: "FSDP: Fully Sharded Data Parallel Training at Scale", checkpointing passage: a local
state dict stores every rank's own shard and can be loaded only with the same number of GPUs and
the same wrapping, while a full state dict gathers the whole model and loads anywhere.  Turning
one rank count's local shards into another's is the operation that lifts that restriction.

Reading used: the source layout is (tensor sizes, pad_src, N_src) and the destination layout is
(the same sizes, pad_dst, N_dst), each flattened and sliced by the floor rule of the page's
sharding passage.  Every tensor's real elements keep their values; destination padding is zero.
The oracle does it the plain way: rebuild each tensor from the source shards, lay the tensors
out again, and cut the destination shards.
"""

import numpy as np

from .layout import flatten_offsets, shard_bounds


def gather_flat(shards):
    """The whole flat vector from its shards in rank order (what a full state dict holds)."""
    return np.concatenate([np.asarray(s) for s in shards]) if len(shards) else np.zeros(0)


def tensors_from_flat(flat, sizes, pad):
    offsets, P = flatten_offsets(sizes, pad)
    assert flat.size == P
    return [flat[o:o + s] for o, s in zip(offsets, sizes)]


def flat_from_tensors(tensors, sizes, pad, dtype):
    offsets, P = flatten_offsets(sizes, pad)
    flat = np.zeros(P, dtype=dtype)
    for o, s, t in zip(offsets, sizes, tensors):
        flat[o:o + s] = t
    return flat


def reshard(shards, sizes, pad_src, pad_dst, n_dst):
    """Destination shards (list of n_dst arrays) from the source shards (list, rank order)."""
    flat = gather_flat(shards)
    dtype = flat.dtype
    tensors = tensors_from_flat(flat, sizes, pad_src)
    out_flat = flat_from_tensors(tensors, sizes, pad_dst, dtype)
    P = out_flat.size
    result = []
    for k in range(n_dst):
        lo, hi = shard_bounds(P, n_dst, k)
        result.append(out_flat[lo:hi].copy())
    return result


def shard(flat_or_tensors, sizes, pad, n, dtype=None):
    """Shards of a flat vector (given either flat or as per-tensor arrays) under (pad, n)."""
    if isinstance(flat_or_tensors, (list, tuple)):
        flat = flat_from_tensors(flat_or_tensors, sizes, pad, dtype)
    else:
        flat = np.asarray(flat_or_tensors)
    P = flat.size
    return [flat[slice(*shard_bounds(P, n, k))].copy() for k in range(n)]
