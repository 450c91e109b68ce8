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
