"""GPU parity of reshard_copy (executing reshard_plan) against the oracle's reshard.

Bit-exact (a copy).  Source shards and the destination carry sentinel guard bands; element
sizes 2, 4 and 8 bytes; world size and padding multiple both change, so pieces start at every
relative 16-byte phase.  The full-size case reshards the 2,000-tensor workload's flat vector from
16 ranks with padding 16 to 12 ranks with padding 12.
"""

import random

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from oracle import layout as OL
from oracle import reshard as OR
from gpu_helpers import Guarded, say

pytestmark = pytest.mark.gpu


def _guarded_raw(host):
    """Guarded buffer for any dtype: viewed as uint16 words (elements are 2, 4 or 8 bytes)."""
    return Guarded(np.ascontiguousarray(host).view(np.uint16))


def _run(sizes, pa, na, pb, nb, dtype, seed):
    offs, Pa = OL.flatten_offsets(sizes, pa)
    rng = np.random.default_rng(seed)
    flat = np.zeros(Pa, dtype=dtype)
    for o, s in zip(offs, sizes):
        flat[o:o + s] = (rng.integers(1, 1 << 15, s)).astype(dtype)
    src = OR.shard(flat, sizes, pa, na)
    want = OR.reshard(src, sizes, pa, pb, nb)
    words = np.dtype(dtype).itemsize // 2
    gsrc = [_guarded_raw(s) for s in src]
    for k in range(nb):
        pieces = F.reshard_plan(sizes, pa, na, pb, nb, k)
        dst = _guarded_raw(np.full(want[k].size, 77, dtype=dtype))
        tdt = {2: torch.int16, 4: torch.float32, 8: torch.float64}[words * 2]
        src_views = [g.data().view(tdt) if g.n else torch.empty(0, dtype=tdt, device="cuda")
                     for g in gsrc]
        F.reshard_copy(src_views, dst.data().view(tdt), pieces)
        torch.cuda.synchronize()
        got = dst.data_host().view(dtype)
        assert np.array_equal(got, want[k]), (sizes, pa, na, pb, nb, k)
        dst.assert_guards("destination")
    for g in gsrc:
        g.assert_guards("source")


@pytest.mark.parametrize("dtype", [np.float32, np.uint16, np.float64])
def test_random_layouts(dtype):
    rng = random.Random({np.float32: 1, np.uint16: 2, np.float64: 3}[dtype])
    for trial in range(25):
        T = rng.randint(1, 9)
        sizes = [rng.choice([1, 2, 3, 5, 8, 17, 100, 1000, 4099, 70001]) for _ in range(T)]
        pa, pb = rng.choice([1, 2, 8, 16]), rng.choice([1, 2, 4, 8, 16])
        na, nb = rng.randint(1, 9), rng.randint(1, 9)
        say(f"reshard trial {trial} T={T} {pa}/{na} -> {pb}/{nb}")
        _run(sizes, pa, na, pb, nb, dtype, trial)


def test_many_pieces_span_several_launches():
    # 400 small tensors with padding changes: several hundred pieces per destination shard,
    # more than one launch's worth.
    sizes = [(i * 37) % 101 + 1 for i in range(400)]
    _run(sizes, 16, 3, 8, 2, np.float32, 7)


@pytest.mark.slow
def test_full_size_many_small_tensors():
    w = W.WORKLOADS["many_small_n16_rank3"]
    sizes = w.sizes
    offs, Pa = OL.flatten_offsets(sizes, 16)
    say(f"full-size reshard P={Pa}")
    codes = np.zeros(Pa, dtype=np.int64)
    for i, (o, s) in enumerate(zip(offs, sizes)):
        codes[o:o + s] = (i << 32) + np.arange(1, s + 1, dtype=np.int64)  # unique, never 0
    src = OR.shard(codes, sizes, 16, 16)
    want = OR.reshard(src, sizes, 16, 12, 12)
    dsrc = [torch.from_numpy(s).cuda() for s in src]
    del codes
    for k in (0, 5, 11):
        pieces = F.reshard_plan(sizes, 16, 16, 12, 12, k)
        dst = torch.full((want[k].size + 8,), 123, dtype=torch.int64, device="cuda")
        F.reshard_copy(dsrc, dst[4:4 + want[k].size], pieces)
        torch.cuda.synchronize()
        h = dst.cpu().numpy()
        assert np.array_equal(h[4:4 + want[k].size], want[k])
        assert (h[:4] == 123).all() and (h[4 + want[k].size:] == 123).all()
        say(f"  rank {k}: {len(pieces)} pieces ok")


def _codes(pos):
    """32-bit code of a flat source position: a multiplicative hash, one-to-one on 32 bits, so a
    misplaced element (by anything other than a multiple of 2**32 positions) shows."""
    return (pos.astype(np.uint64) * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)


@pytest.mark.slow
@pytest.mark.parametrize("dst_pad,dst_world,dst_rank", [(1, 6, 1), (16, 6, 5), (8, 12, 0)])
def test_full_size_dense7b_sampled(dst_pad, dst_world, dst_rank):
    # The 7B-shaped model's fp32 state from 8 ranks (padding 1) to another layout, as the bench
    # times it.  Source shards hold the hashed source flat position of each element; sampled
    # destination elements (every piece boundary and 1M random positions) are checked against
    # the position the oracle's flat layout gives them.
    w = W.WORKLOADS["dense7b_n8_rank0"]
    sizes, pa, na = w.sizes, w.pad_multiple, w.world_size
    offs_a, Pa = OL.flatten_offsets(sizes, pa)
    offs_b, Pb = OL.flatten_offsets(sizes, dst_pad)
    lo_b, hi_b = OL.shard_bounds(Pb, dst_world, dst_rank)
    n_dst = hi_b - lo_b
    pieces = F.reshard_plan(sizes, pa, na, dst_pad, dst_world, dst_rank)
    used = sorted({int(r) for r in pieces["src_rank"] if r >= 0})
    say(f"dense7b reshard {na}/{pa} -> {dst_world}/{dst_pad} rank {dst_rank}: n={n_dst} "
        f"pieces={len(pieces)} sources={used}")
    src = []
    for r in range(na):
        if r not in used:
            src.append(None)
            continue
        lo, hi = OL.shard_bounds(Pa, na, r)
        t = torch.empty(hi - lo, dtype=torch.int32, device="cuda")
        step = 1 << 27
        for a in range(lo, hi, step):
            b = min(hi, a + step)
            pos = torch.arange(a, b, dtype=torch.int64, device="cuda")
            t[a - lo:b - lo] = ((pos * 2654435761) & 0xFFFFFFFF).to(torch.int32)
        src.append(t)
    dst = torch.full((n_dst + 8,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    F.reshard_copy(src, dst[4:4 + n_dst], pieces)
    torch.cuda.synchronize()

    rng = np.random.default_rng(dst_rank)
    bounds = np.concatenate([pieces["dst_offset"], pieces["dst_offset"] + pieces["length"]])
    near = (bounds[:, None] + np.arange(-3, 3)[None, :]).reshape(-1)
    j = np.unique(np.concatenate([near, rng.integers(0, n_dst, 1 << 20), [0, n_dst - 1]]))
    j = j[(j >= 0) & (j < n_dst)]
    q = lo_b + j                                       # flat position in the destination layout
    ob = np.asarray(offs_b + [Pb], dtype=np.int64)
    oa = np.asarray(offs_a, dtype=np.int64)
    ti = np.searchsorted(ob, q, side="right") - 1
    off = q - ob[ti]
    real = off < np.asarray(sizes, dtype=np.int64)[ti]
    want = np.where(real, _codes(oa[ti] + off), 0).astype(np.uint32)
    got = dst[4:4 + n_dst][torch.from_numpy(j).cuda()].cpu().numpy().view(np.uint32)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (j[bad[:5]], got[bad[:5]], want[bad[:5]])
    guard = torch.cat([dst[:4], dst[4 + n_dst:]]).cpu().numpy()
    assert (guard == 0x5A5A5A5A).all()
    say(f"  {j.size} sampled elements ok ({int(real.sum())} real)")


@pytest.mark.slow
def test_full_state_dict_from_2000_tensor_shards():
    """16 ranks with padding 16 -> one rank without padding: the result must be every tensor's
    values back to back, which is what a full (unsharded, unpadded) state dict holds.  Each real
    element carries its running index + 1 and padding carries 0, so the expected vector is
    1..P_real by definition, with no call to the oracle's reshard."""
    w = W.WORKLOADS["many_small_n16_rank3"]
    sizes, pa, na = w.sizes, w.pad_multiple, w.world_size
    offs, Pa = OL.flatten_offsets(sizes, pa)
    real_total = int(np.sum(sizes))
    flat = np.zeros(Pa, dtype=np.int32)
    start = 1
    for o, s in zip(offs, sizes):
        flat[o:o + s] = np.arange(start, start + s, dtype=np.int32)
        start += s
    src = []
    for k in range(na):
        lo, hi = OL.shard_bounds(Pa, na, k)
        src.append(torch.from_numpy(flat[lo:hi].copy()).cuda())
    del flat
    pieces = F.reshard_plan(sizes, pa, na, 1, 1, 0)
    say(f"full state dict: {na}/{pa} -> 1/1, {real_total} elements, {len(pieces)} pieces")
    dst = torch.full((real_total + 8,), -7, dtype=torch.int32, device="cuda")
    F.reshard_copy(src, dst[4:4 + real_total], pieces)
    want = torch.arange(1, real_total + 1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    assert torch.equal(dst[4:4 + real_total], want)
    h = dst.cpu().numpy()
    assert (h[:4] == -7).all() and (h[4 + real_total:] == -7).all()
    del src, dst, want
    torch.cuda.empty_cache()
