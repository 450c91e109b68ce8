"""The step calls inside a captured HIP graph.

The library allocates nothing, issues no memset and never synchronises, so a caller can capture
its calls.  Captured here: the global-norm sum of squares of the gradient contributions (two
kernels, workspace from the binding) followed by the clipped blocked-state step; the same with
the contributions interleaved in one array; and, separately, the fp32-gradient path (reduction
fused with its sum of squares, then the clipped fp32-gradient step).  The graph is replayed several times, with eager work and synchronisation between the
replays, and after every replay its buffers must equal, bit for bit, those of the same calls
run eagerly on a second copy of the inputs.
"""

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from gpu_helpers import bit_equal, say, to_dev16

pytestmark = pytest.mark.gpu

SIZES, PAD, WD, N, K = [5000, 3, 12000, 1, 7777, 40001, 65536], 16, [1, 0, 1, 1, 0, 1, 1], 3, 1
REPLAYS = 4


def _setup(seed):
    L, segs = F.shard_layout(SIZES, N, K, PAD, WD)
    n = L.n
    master = torch.from_numpy(W.np_f32_normal([seed, 1], n, 0.02)).cuda()
    m = torch.from_numpy(W.np_f32_normal([seed, 2], n, 1e-3)).cuda()
    v = (torch.from_numpy(W.np_f32_normal([seed, 3], n, 1e-3)).cuda() ** 2).contiguous()
    state = torch.zeros(F.state_blocked_elems(n), dtype=torch.float32, device="cuda")
    F.state_to_blocked(master, m, v, state)
    grads = [to_dev16(W.np_bf16_normal([seed, 4, r], n, 1e-2)) for r in range(4)]
    gi = torch.empty(F.grads_interleaved_elems(4, n), dtype=torch.int16, device="cuda")
    F.grads_to_interleaved(grads, gi, n=n)
    torch.cuda.synchronize()
    return L, F.segments_to_device(segs), state, (grads, gi)


def _buffers(L, state):
    phase = L.lo % 8
    return dict(state=state.clone(),
                flat=torch.zeros(L.n + phase, dtype=torch.int16, device="cuda"),
                sumsq=torch.zeros(1, dtype=torch.float64, device="cuda"),
                acc=torch.zeros(L.n, dtype=torch.float32, device="cuda"))


def _run(path, L, sd, inputs, b):
    """One step on the buffers in `b`, enqueued on the current stream."""
    grads, gi = inputs
    phase = L.lo % 8
    kw = dict(step=3, lr=1e-3, weight_decay=0.01, segs=sd, n_segments=L.n_segments,
              flat=b["flat"], flat_index0=L.lo - phase, lo=L.lo, max_grad_norm=0.05,
              grad_sumsq=b["sumsq"])
    if path == "bf16":
        F.grad_sumsq_shard(b["sumsq"], contribs=grads, n=L.n, segs=sd, n_segments=L.n_segments)
        F.adamw_shard_step_blocked(b["state"], grads, n=L.n, **kw)
    elif path == "interleaved":
        F.grad_sumsq_shard_interleaved(b["sumsq"], gi, len(grads), L.n, segs=sd,
                                       n_segments=L.n_segments)
        F.adamw_shard_step_interleaved(b["state"], gi, len(grads), n=L.n, **kw)
    else:
        F.reduce_shard_sumsq(grads, b["acc"], b["sumsq"], n=L.n, segs=sd,
                             n_segments=L.n_segments)
        F.adamw_shard_step_f32grad_blocked(b["state"], b["acc"], n=L.n, **kw)


def _host(b):
    return {k: t.cpu().numpy() for k, t in b.items()}


@pytest.mark.parametrize("path", ["bf16", "interleaved", "f32"])
def test_graph_replays_match_eager(path):
    L, sd, state0, inputs = _setup(321)
    say(f"graph capture, {path} path: n={L.n} lo={L.lo} segments={L.n_segments}")
    eager = _buffers(L, state0)
    graphed = _buffers(L, state0)
    warm = _buffers(L, state0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(path, L, sd, inputs, warm)         # warm-up on a side stream, on its own buffers
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(path, L, sd, inputs, graphed)
    torch.cuda.synchronize()
    # Capture records the kernels without running them: the buffers still hold the inputs.
    assert bit_equal(graphed["state"].cpu().numpy(), state0.cpu().numpy())

    for rep in range(REPLAYS):
        _run(path, L, sd, inputs, eager)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        torch.randn(1 << 20, device="cuda").sum()          # unrelated eager work in between
        torch.cuda.synchronize()
        got, want = _host(graphed), _host(eager)
        for key in ("state", "flat", "sumsq") + (("acc",) if path == "f32" else ()):
            if key == "sumsq":
                assert got[key].view(np.uint64)[0] == want[key].view(np.uint64)[0], \
                    f"replay {rep}: sumsq"
            else:
                assert bit_equal(got[key], want[key]), f"replay {rep}: {key}"
        say(f"  replay {rep} equals the eager step")
    # The replays moved the state: each one is a real step.
    assert not bit_equal(graphed["state"].cpu().numpy(), state0.cpu().numpy())
