"""The measurement aids write exactly what include/fsdpshard_calib.h says, on ragged sizes (a
last work-group only partly inside the streams), so their bandwidth figures come from kernels
that touch every byte they claim and nothing else."""

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_layout_amd as F
import blocked_layout as BL
from gpu_helpers import say

pytestmark = pytest.mark.gpu
GUARD = 64


def _dev_u32(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int32)).cuda()


def _index_pattern(nvec):
    i = np.arange(nvec, dtype=np.uint32)
    return np.stack([i, i ^ np.uint32(0x55555555), i ^ np.uint32(0x33333333),
                     i ^ np.uint32(0x0F0F0F0F)], axis=1)


@pytest.mark.parametrize("n_src,n_dst", [(1, 1), (2, 1), (0, 2), (3, 2)])
@pytest.mark.parametrize("vpt,threads,per_cu,run", [(4, 256, 0, 0), (1, 1024, 2, 1), (2, 512, 0, 4),
                                                    (4, 256, 1, 2)])
def test_stream_rw_writes_what_it_reads(n_src, n_dst, vpt, threads, per_cu, run):
    nvec = 8192 * 11 + 333                      # many work-groups, the last one partial
    nbytes = nvec * 16
    rng = np.random.default_rng(n_src * 10 + n_dst)
    srcs = [rng.integers(0, 2 ** 32, (nvec, 4), dtype=np.uint32) for _ in range(n_src)]
    dsts = [np.full((nvec + GUARD, 4), 0xA5A5A5A5, dtype=np.uint32) for _ in range(n_dst)]
    sd = [_dev_u32(s) for s in srcs]
    dd = [_dev_u32(d) for d in dsts]
    say(f"stream_rw {n_src} read, {n_dst} write streams, {nvec} vectors, shape "
        f"{vpt}/{threads}/{per_cu}/{run}")
    F.stream_rw(sd, dd, nbytes, vectors_per_thread=vpt, threads_per_group=threads, per_cu=per_cu,
                xcd_run=run)
    torch.cuda.synchronize()
    want = _index_pattern(nvec)
    for s in srcs:
        want = want ^ s
    for w, d in enumerate(dd):
        got = d.cpu().numpy().view(np.uint32).reshape(-1, 4)
        exp = want.copy()
        exp[:, 0] += np.uint32(w)
        assert np.array_equal(got[:nvec], exp), f"destination {w}"
        assert (got[nvec:] == 0xA5A5A5A5).all(), f"destination {w}: guard written"
    for s, d in zip(srcs, sd):
        assert np.array_equal(d.cpu().numpy().view(np.uint32).reshape(-1, 4), s)


@pytest.mark.parametrize("n_src", [1, 2])
@pytest.mark.parametrize("vpt,threads,per_cu,run", [(4, 256, 0, 0), (2, 512, 2, 32)])
def test_stream_rw_in_place(n_src, vpt, threads, per_cu, run):
    """A write stream that is also a read stream (the last one): it receives the XOR of the
    sources as they were before the call, and nothing past the stream changes."""
    nvec = 8192 * 11 + 333
    nbytes = nvec * 16
    rng = np.random.default_rng(70 + n_src)
    srcs = [rng.integers(0, 2 ** 32, (nvec + GUARD, 4), dtype=np.uint32) for _ in range(n_src)]
    sd = [_dev_u32(s) for s in srcs]
    say(f"stream_rw in place, {n_src} read streams, shape {vpt}/{threads}/{per_cu}/{run}")
    F.stream_rw(sd, [sd[-1]], nbytes, vectors_per_thread=vpt, threads_per_group=threads,
                per_cu=per_cu, xcd_run=run)
    torch.cuda.synchronize()
    want = _index_pattern(nvec)
    for s in srcs:
        want = want ^ s[:nvec]
    got = sd[-1].cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.array_equal(got[:nvec], want)
    assert np.array_equal(got[nvec:], srcs[-1][nvec:]), "past the stream written"
    for s, d in zip(srcs[:-1], sd[:-1]):
        assert np.array_equal(d.cpu().numpy().view(np.uint32).reshape(-1, 4), s)


def test_stream_rw_pure_reads_leave_the_sink():
    nvec = 4096 + 17
    src = _dev_u32(np.ones((nvec, 4), dtype=np.uint32))
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    F.stream_rw([src], [], nvec * 16, sink=sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def _mix_expected(contribs, state, n, shaped):
    """What the replicas write: per 8-element vector, x = XOR of the contributions' words (and,
    for the shaped replica, of every state word but each array's first); the state's first word
    of each array XOR x; out = (master[1], m[1], v[1], x) of the vector."""
    nvec = n // 8
    x = np.zeros(nvec, dtype=np.uint32)
    for c in contribs:
        x ^= np.bitwise_xor.reduce(c.view(np.uint32).reshape(nvec, 4), axis=1)
    sep = [a.view(np.uint32).reshape(nvec, 8).copy() for a in BL.from_blocked(state, n)]
    if shaped:
        for a in sep:
            x ^= np.bitwise_xor.reduce(a[:, 1:], axis=1)
    out = np.stack([sep[0][:, 1], sep[1][:, 1], sep[2][:, 1], x], axis=1)
    for a in sep:
        a[:, 0] ^= x
    return [a.reshape(-1).view(np.float32) for a in sep], out


@pytest.mark.parametrize("fan_in", [1, 8])
@pytest.mark.parametrize("groups,per_cu,run,phased", [(0, 0, 0, 0), (1, 2, 32, 1), (2, 1, 2, 1),
                                                      (4, 1, 1, 1), (1, 1, 16, 0), (2, 2, 4, 0),
                                                      (-1, 0, 0, 0)])
def test_mix_replicas_move_the_steps_bytes(fan_in, groups, per_cu, run, phased):
    # groups -1: the replica of the step fed by interleaved contributions.
    n = 8 * (64 * 4 * 4 * 21 + 97)               # 21 whole tiles of 16 groups plus a ragged tail
    rng = np.random.default_rng(fan_in + groups)
    contribs = [rng.integers(0, 2 ** 16, n, dtype=np.uint16) for _ in range(fan_in)]
    sep = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    unused = np.uint32(0x7FB0B0B0).view(np.float32)
    state = BL.to_blocked(*sep, fill=unused)
    st = torch.from_numpy(np.concatenate([state, np.full(GUARD, unused, np.float32)])).cuda()
    out = torch.full((2 * n // 2 + GUARD,), 0x5A5A, dtype=torch.int16, device="cuda")
    cd = [torch.from_numpy(c.view(np.int16)).cuda() for c in contribs]
    say(f"mix replica fan-in {fan_in} groups {groups} per_cu {per_cu} run {run} phased {phased} "
        f"n={n}")
    if groups == 0:
        F.stream_mix_blocked(cd, st, out, n)
    elif groups == -1:
        gi = torch.from_numpy(BL.to_interleaved(contribs).view(np.int16)).cuda()
        F.stream_mix_interleaved(gi, fan_in, st, out, n)
    else:
        F.stream_mix_shaped(cd, st, out, n, groups, per_cu, run, phased)
    torch.cuda.synchronize()
    want_sep, want_out = _mix_expected(contribs, state, n, shaped=groups > 0)
    got = st.cpu().numpy()
    for k, (g, w) in enumerate(zip(BL.from_blocked(got[:state.size], n), want_sep)):
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"state array {k}"
    assert (got[state.size:].view(np.uint32) == 0x7FB0B0B0).all(), "state guard written"
    used = BL.to_blocked(*(np.ones(n, np.float32) for _ in range(3)), fill=0.0) != 0.0
    assert (got[:state.size][~used].view(np.uint32) == 0x7FB0B0B0).all(), "unused slots written"
    o = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(o[:n].view(np.uint32).reshape(-1, 4), want_out)
    assert (o[n:] == 0x5A5A).all(), "out guard written"
