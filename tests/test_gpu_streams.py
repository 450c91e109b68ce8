"""Stream ordering through the binding: every call enqueues on the stream it is given.

* The clipped paths (sum of squares, then the step that reads it; with the contributions in
  separate arrays and interleaved in one) run on a side stream and give bit for bit the results
  of the same calls on the current stream.  The bindings allocate the
  sums' workspace themselves here, and the current stream allocates and writes while the side
  stream's kernels are still queued: the workspace must stay reserved for the side stream.
* Two slices of one layout stepped concurrently on two streams equal the same steps run one
  after the other.
All streams have the default priority.
"""

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from gpu_helpers import say, to_dev16

pytestmark = pytest.mark.gpu
HP = dict(W.ADAMW)


def _blocked(master):
    n = master.numel()
    # Zeroed: the slots past n in the last block are never written and would otherwise keep
    # whatever the allocator's block held.
    st = torch.zeros(F.state_blocked_elems(n), dtype=torch.float32, device="cuda")
    F.state_to_blocked(master, torch.zeros_like(master), torch.zeros_like(master), st)
    return st


def _clipped_paths(dev, gi, master, n, stream):
    """Clipped bf16-contribution step and clipped fp32-gradient step, both blocked, from the
    separate contributions `dev` and from their interleaved array `gi`; returns the states, the
    bf16 outputs and the sums."""
    fan_in = len(dev)
    st1, st2, st3, st4 = (_blocked(master) for _ in range(4))
    out1, out2, out3, out4 = (torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(4))
    g32 = torch.empty(n, dtype=torch.float32, device="cuda")
    g32i = torch.empty(n, dtype=torch.float32, device="cuda")
    sq1, sq2, sq3, sq4 = (torch.zeros(1, dtype=torch.float64, device="cuda") for _ in range(4))
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())
    F.grad_sumsq_shard(sq1, contribs=dev, n=n, stream=stream)
    F.adamw_shard_step_blocked(st1, dev, step=1, n=n, flat=out1, max_grad_norm=0.05,
                               grad_sumsq=sq1, stream=stream, **HP)
    F.reduce_shard_sumsq(dev, g32, sq2, stream=stream)
    F.adamw_shard_step_f32grad_blocked(st2, g32, step=1, n=n, flat=out2, max_grad_norm=0.05,
                                       grad_sumsq=sq2, stream=stream, **HP)
    F.grad_sumsq_shard_interleaved(sq3, gi, fan_in, n, stream=stream)
    F.adamw_shard_step_interleaved(st3, gi, fan_in, step=1, n=n, flat=out3, max_grad_norm=0.05,
                                   grad_sumsq=sq3, stream=stream, **HP)
    F.reduce_shard_sumsq_interleaved(gi, fan_in, g32i, sq4, stream=stream)
    F.adamw_shard_step_f32grad_blocked(st4, g32i, step=1, n=n, flat=out4, max_grad_norm=0.05,
                                       grad_sumsq=sq4, stream=stream, **HP)
    if stream is not None:
        # Allocate and write on the current stream while the side stream's work is queued
        # (small blocks, the size class of the sums' workspace, and large ones).
        junk = [torch.full((64,), float("nan"), device="cuda") for _ in range(256)]
        junk += [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(4)]
        del junk
        stream.synchronize()
    torch.cuda.synchronize()
    return st1, st2, st3, st4, out1, out2, out3, out4, sq1, sq2, sq3, sq4


@pytest.mark.parametrize("F_in", [8, 4])
def test_side_stream_matches_current_stream(F_in):
    n = 1_000_003
    say(f"side stream, clipped paths, F={F_in} n={n}")
    contribs = [W.np_bf16_normal([95, r], n, 1e-2) for r in range(F_in)]
    dev = [to_dev16(c) for c in contribs]
    gi = torch.empty(F.grads_interleaved_elems(F_in, n), dtype=torch.int16, device="cuda")
    F.grads_to_interleaved(dev, gi, n=n)
    master = torch.from_numpy(W.np_f32_normal([96, 0], n, 0.02)).cuda()
    want = _clipped_paths(dev, gi, master, n, None)
    side = torch.cuda.Stream()
    got = _clipped_paths(dev, gi, master, n, side)
    names = ("state", "state f32", "state interleaved", "state interleaved f32", "bf16",
             "bf16 f32", "bf16 interleaved", "bf16 interleaved f32", "sumsq", "sumsq f32",
             "sumsq interleaved", "sumsq interleaved f32")
    for a, b, what in zip(got, want, names):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what
    # The two layouts agree with each other as well.
    for i, j in ((0, 2), (1, 3), (4, 6), (5, 7), (8, 10), (9, 11)):
        assert torch.equal(want[i].view(torch.uint8), want[j].view(torch.uint8)), names[j]
    assert float(want[8].item()) > 0.0


def test_two_streams_step_disjoint_slices():
    sizes = [(i * 7919) % 3001 + 1 for i in range(300)]
    N, F_in = 4, 8
    say(f"two streams, two ranks of {N}")
    runs = {}
    for mode in ("sequential", "concurrent"):
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        res = []
        for k, s in zip((1, 2), streams):
            L, segs = F.shard_layout(sizes, N, k, 16, [i % 2 == 0 for i in range(300)])
            sd = F.segments_to_device(segs)
            dev = [to_dev16(W.np_bf16_normal([97, k, r], L.n, 1e-2)) for r in range(F_in)]
            st = _blocked(torch.from_numpy(W.np_f32_normal([98, k], L.n, 0.02)).cuda())
            out = torch.zeros(L.n, dtype=torch.int16, device="cuda")
            res.append((L, sd, dev, st, out))
        torch.cuda.synchronize()
        for (L, sd, dev, st, out), s in zip(res, streams):
            s.wait_stream(torch.cuda.current_stream())
            for t in (1, 2, 3):
                F.adamw_shard_step_blocked(st, dev, step=t, n=L.n, segs=sd,
                                           n_segments=L.n_segments, flat=out, flat_index0=L.lo,
                                           lo=L.lo, stream=s, **HP)
            if mode == "sequential":
                s.synchronize()
        torch.cuda.synchronize()
        runs[mode] = [(st.clone(), out.clone()) for (_, _, _, st, out) in res]
    for (a_st, a_out), (b_st, b_out) in zip(runs["sequential"], runs["concurrent"]):
        assert torch.equal(a_st.view(torch.int32), b_st.view(torch.int32))
        assert torch.equal(a_out, b_out)
