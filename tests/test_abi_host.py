"""Host-side checks of the C-ABI library (no GPU needed).

* The library loads and exports every function that include/*.h declares.
* shard_layout (host code in the library) matches the oracle's layout bit for bit, including
  empty shards, padding, the 2,000-tensor workload and the capacity two-call pattern.
* Argument validation returns its status before any HIP call (only calls that stop in
  validation are made here; nothing reaches a kernel launch).
"""

import ctypes
import os
import random
import re

import numpy as np
import pytest

import fsdp_sharded_optimizer_layout_amd as F
import workloads as W
from oracle import layout as OL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, OVERFLOW, CAPACITY, ALIGN, UNSUP, HIPERR = range(7)


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[\w ]+?\**\s*\b(\w+)\s*\(", text, flags=re.M)
    return [n for n in names if n not in ("defined",)]


def test_library_exports_every_declared_symbol():
    lib = F.lib()
    declared = _declared_functions()
    assert {"shard_layout", "reduce_shard", "adamw_shard_step", "unflatten_bf16"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name
    assert F.abi_version() == 1
    assert F.strerror(CAPACITY) == "output array or workspace too small"


def _oracle_segments(sizes, pad, wd, N, k):
    lo, hi, segs = OL.segments(sizes, pad, wd, N, k)
    return lo, hi, [(s["shard_begin"], s["length"], s["tensor_offset"], s["tensor_id"], s["flags"])
                    for s in segs]


def _lib_segments(sizes, pad, wd, N, k):
    L, segs = F.shard_layout(sizes, N, k, pad, wd)
    return L, [tuple(int(x) for x in s) for s in segs]


def test_layout_matches_oracle_random():
    rng = random.Random(3)
    for trial in range(500):
        T = rng.randint(0, 12)
        sizes = [rng.choice([0, 1, 2, 3, 7, 8, 15, 16, 17, 100]) for _ in range(T)]
        pad = rng.choice([1, 2, 8, 16])
        wd = [rng.random() < 0.5 for _ in range(T)] if rng.random() < 0.5 else None
        N = rng.randint(1, 20)
        for k in range(N):
            lo, hi, want = _oracle_segments(sizes, pad, wd, N, k)
            L, got = _lib_segments(sizes, pad, wd, N, k)
            assert (L.lo, L.hi, L.n) == (lo, hi, hi - lo)
            assert got == want
            assert L.n_real == sum(s[1] for s in want if not s[4] & OL.PADDING)


@pytest.mark.parametrize("name", W.ORDER)
def test_layout_of_workloads(name):
    w = W.WORKLOADS[name]
    lo, hi, want = _oracle_segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    L, got = _lib_segments(w.sizes, w.pad_multiple, w.wd_mask, w.world_size, w.rank)
    assert (L.P, L.lo, L.hi) == (w.total, lo, hi)
    assert got == want


def test_workload_realisations():
    # flat lengths and slices of the five shard configurations
    expect = {
        "p1000003_n8_rank3": (1_000_003, 375_001, 500_001),
        "llama_layer_n8_rank0": (218_112_000, 0, 27_264_000),
        "dense7b_n8_rank0": (7_241_728_000, 0, 905_216_000),
        "dense70b_n64_rank0": (68_976_640_000, 0, 1_077_760_000),
        "many_small_n16_rank3": (529_512_096, 99_283_518, 132_378_024),
    }
    for name, (P, lo, hi) in expect.items():
        w = W.WORKLOADS[name]
        L, segs = F.shard_layout(w.sizes, w.world_size, w.rank, w.pad_multiple, w.wd_mask)
        assert (L.P, L.lo, L.hi) == (P, lo, hi)
    L, segs = F.shard_layout(W.WORKLOADS["many_small_n16_rank3"].sizes, 16, 3, 16,
                             W.WORKLOADS["many_small_n16_rank3"].wd_mask)
    assert L.n - L.n_real == 1008 and L.n_real == 33_093_498


def test_empty_shards_when_P_below_N():
    bounds = [F.shard_layout([3], 8, k)[0] for k in range(8)]
    assert [b.lo for b in bounds] + [3] == [0, 0, 0, 1, 1, 1, 2, 2, 3]
    assert [b.n for b in bounds] == [0, 0, 1, 0, 0, 1, 0, 1]
    L, segs = F.shard_layout([], 4, 2)
    assert L.P == 0 and L.n == 0 and segs.size == 0


def test_capacity_two_call_pattern():
    lib = F.lib()
    sizes = (ctypes.c_int64 * 5)(5, 6, 7, 8, 9)
    out = F._Layout()
    segs = (F._Segment * 2)()
    rc = lib.shard_layout(sizes, 5, 4, None, 1, 0, ctypes.byref(out), segs, 2)
    assert rc == CAPACITY and out.n_segments == 9     # tensor 3 (8 elements) has no padding
    assert (segs[0].shard_begin, segs[0].length, segs[1].flags) == (0, 5, 3)
    segs = (F._Segment * 9)()
    assert lib.shard_layout(sizes, 5, 4, None, 1, 0, ctypes.byref(out), segs, 9) == OK


def test_layout_argument_errors():
    lib = F.lib()
    sizes = (ctypes.c_int64 * 2)(5, 6)
    out = F._Layout()
    assert lib.shard_layout(sizes, 2, 1, None, 0, 0, ctypes.byref(out), None, 0) == INVALID
    assert lib.shard_layout(sizes, 2, 1, None, 4, 4, ctypes.byref(out), None, 0) == INVALID
    assert lib.shard_layout(sizes, 2, 1, None, 4, -1, ctypes.byref(out), None, 0) == INVALID
    assert lib.shard_layout(sizes, 2, 0, None, 4, 0, ctypes.byref(out), None, 0) == INVALID
    assert lib.shard_layout(None, 2, 1, None, 4, 0, ctypes.byref(out), None, 0) == INVALID
    assert lib.shard_layout(sizes, 2, 1, None, 4, 0, None, None, 0) == INVALID
    neg = (ctypes.c_int64 * 1)(-1)
    assert lib.shard_layout(neg, 1, 1, None, 4, 0, ctypes.byref(out), None, 0) == INVALID
    big = (ctypes.c_int64 * 2)(2 ** 62, 2 ** 62)
    assert lib.shard_layout(big, 2, 1, None, 4, 0, ctypes.byref(out), None, 0) == OVERFLOW
    odd = (ctypes.c_int64 * 1)(2 ** 63 - 5)
    assert lib.shard_layout(odd, 1, 16, None, 4, 0, ctypes.byref(out), None, 0) == OVERFLOW


def test_layout_128bit_product():
    # k * P overflows int64 for P near 2^62 and k = 63; the library forms it in 128 bits.
    P = 2 ** 62 + 12345
    for k in (1, 31, 63):
        L, _ = F.shard_layout([P], 64, k)
        assert (L.lo, L.hi) == OL.shard_bounds(P, 64, k)


class _Fake:
    """Aligned fake device addresses: only used for calls that stop in argument validation."""
    base = 1 << 40

    @classmethod
    def at(cls, i, off=0):
        return cls.base + i * (1 << 32) + off


def _step(lib, master, m, v, contribs, fan_in, n, segs, nseg, hp, flat, f0, lo):
    arr = (ctypes.c_void_p * max(1, len(contribs)))(*contribs) if contribs is not None else None
    return lib.adamw_shard_step(master, m, v, arr, fan_in, n, segs, nseg,
                                ctypes.byref(hp) if hp is not None else None, flat, f0, lo, None)


def test_step_validation_errors():
    lib = F.lib()
    hp = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    a, b, c = _Fake.at(0), _Fake.at(1), _Fake.at(2)
    g = [_Fake.at(3), _Fake.at(4)]
    out = _Fake.at(5)
    # n == 0 with valid arguments: success without touching the GPU
    assert _step(lib, a, b, c, g, 2, 0, None, 0, hp, out, 0, 0) == OK
    assert _step(lib, None, b, c, g, 2, 0, None, 0, hp, out, 0, 0) == INVALID
    assert _step(lib, a, b, c, g, 2, -1, None, 0, hp, out, 0, 0) == INVALID
    assert _step(lib, a, b, c, g, 0, 0, None, 0, hp, out, 0, 0) == INVALID
    assert _step(lib, a, b, c, g * 40, 65, 0, None, 0, hp, out, 0, 0) == UNSUP
    assert _step(lib, a, b, c, [g[0], None], 2, 0, None, 0, hp, out, 0, 0) == INVALID
    assert _step(lib, a, b, c, [g[0], g[1] + 2], 2, 0, None, 0, hp, out, 0, 0) == ALIGN
    assert _step(lib, a + 4, b, c, g, 2, 0, None, 0, hp, out, 0, 0) == ALIGN
    assert _step(lib, a, b, c, g, 2, 0, None, 0, hp, out + 1, 0, 0) == ALIGN
    assert _step(lib, a, b, c, g, 2, 0, _Fake.at(6, 4), 1, hp, out, 0, 0) == ALIGN
    assert _step(lib, a, b, c, g, 2, 0, None, 3, hp, out, 0, 0) == INVALID   # count without table
    assert _step(lib, a, b, c, g, 2, 0, None, 0, hp, out, 5, 4) == INVALID   # window after lo
    assert _step(lib, a, b, c, g, 2, 0, None, 0, None, out, 0, 0) == INVALID
    for bad in (dict(step=0), dict(beta1=1.0), dict(beta2=-0.1), dict(lr=float("nan")),
                dict(eps=float("inf"))):
        h = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
        for k, val in bad.items():
            setattr(h, k, val)
        assert _step(lib, a, b, c, g, 2, 0, None, 0, h, out, 0, 0) == INVALID
    # overlapping written buffers are refused (checked when n > 0, before any launch)
    assert _step(lib, a, a + 16, c, g, 2, 100, None, 0, hp, out, 0, 0) == INVALID
    assert _step(lib, a, b, c, [a, g[1]], 2, 100, None, 0, hp, out, 0, 0) == INVALID
    assert _step(lib, a, b, c, g, 2, 100, None, 0, hp, g[0] + 64, 0, 0) == INVALID


def test_interleaved_validation_errors():
    """The interleaved gradient array: its size rule, and every argument check of the step and of
    the conversion, which stop before anything is launched."""
    lib = F.lib()
    assert F.grads_interleaved_elems(8, 1000) == 8 * 1024
    assert F.grads_interleaved_elems(3, 512) == 3 * 512
    assert F.grads_interleaved_elems(1, 0) == 0
    assert lib.grads_interleaved_elems(0, 10) == -1
    assert lib.grads_interleaved_elems(65, 10) == -1
    assert lib.grads_interleaved_elems(2, -1) == -1
    assert lib.grads_interleaved_elems(64, 2 ** 62) == -1          # bytes beyond int64
    hp = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    st, gi, out = _Fake.at(0), _Fake.at(1), _Fake.at(2)
    il = lambda state, grads, fan_in, n, segs=None, nseg=0, h=hp, flat=out: \
        lib.adamw_shard_step_interleaved(state, grads, fan_in, n, segs, nseg,
                                         ctypes.byref(h) if h is not None else None, flat, 0, 0,
                                         None)
    assert il(st, gi, 8, 0) == OK
    assert il(st, None, 8, 0) == INVALID
    assert il(None, gi, 8, 0) == INVALID
    assert il(st, gi, 0, 0) == INVALID
    assert il(st, gi, 65, 0) == UNSUP
    assert il(st, gi + 8, 8, 0) == ALIGN
    assert il(st + 4, gi, 8, 0) == ALIGN
    assert il(st, gi, 8, -1) == INVALID
    assert il(st, gi, 8, 0, h=None) == INVALID
    assert il(st, gi, 64, 2 ** 59) == OVERFLOW
    n = 1000                                  # 8 * 1024 bf16 = 16 KiB of gradients
    assert il(st, gi, 8, n, flat=gi + 16384 - 64) == INVALID       # bf16 window inside grads
    assert il(gi + 16384 - 16, gi, 8, n) == INVALID                # state over the grads' end
    assert il(st, gi, 8, n, segs=st + 64, nseg=1) == INVALID       # table inside the state
    clip = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1, 1.0, st + 8)
    assert il(st, gi, 8, n, h=clip) == INVALID                     # sum inside the state
    g = (ctypes.c_void_p * 2)(_Fake.at(3), _Fake.at(4))
    conv = lib.grads_to_interleaved
    assert conv(g, 2, 0, gi, None) == OK
    assert conv(g, 2, 0, None, None) == INVALID
    assert conv(g, 0, 0, gi, None) == INVALID
    assert conv(g, 2, -1, gi, None) == INVALID
    assert conv(g, 2, 0, gi + 2, None) == ALIGN
    assert conv((ctypes.c_void_p * 2)(_Fake.at(3), None), 2, 0, gi, None) == INVALID
    # the 2 * 512-element array (2 KiB) starting 1 KiB before a contribution runs into it
    assert conv(g, 2, 100, _Fake.at(3, -1024), None) == INVALID
    assert conv(g, 2, 100, _Fake.at(4, -1024), None) == INVALID
    sq = lambda grads, fan_in, n, segs=None, nseg=0, ws=_Fake.at(7), wsb=1 << 20, res=_Fake.at(8): \
        lib.grad_sumsq_shard_interleaved(grads, fan_in, n, segs, nseg, 1.0, ws, wsb, res, None)
    # (n == 0 still launches the kernel that writes +0 into sumsq, so no call below succeeds)
    assert sq(None, 8, 0) == INVALID
    assert sq(gi, 0, 0) == INVALID
    assert sq(gi, 65, 0) == UNSUP
    assert sq(gi + 8, 8, 0) == ALIGN
    assert sq(gi, 8, 0, res=None) == INVALID
    assert sq(gi, 8, -1) == INVALID
    assert sq(gi, 64, 2 ** 59) == OVERFLOW
    assert sq(gi, 8, n, wsb=0) == CAPACITY
    assert sq(gi, 8, n, ws=gi + 16384 - 8) == INVALID          # workspace over the grads' end
    assert sq(gi, 8, n, res=gi + 8192) == INVALID              # sum inside the grads
    assert sq(gi, 8, n, segs=_Fake.at(7), nseg=1) == INVALID     # table over the workspace
    red = lambda grads, fan_in, n, out=_Fake.at(9), acc=0: \
        lib.reduce_shard_interleaved(grads, fan_in, n, 1.0, out, acc, None)
    assert red(gi, 8, 0) == OK
    assert red(None, 8, 0) == INVALID
    assert red(gi, 8, 0, out=None) == INVALID
    assert red(gi, 0, 0) == INVALID
    assert red(gi, 65, 0) == UNSUP
    assert red(gi + 8, 8, 0) == ALIGN
    assert red(gi, 8, 0, out=_Fake.at(9, 8)) == ALIGN
    assert red(gi, 8, 0, acc=2) == INVALID
    assert red(gi, 64, 2 ** 59) == OVERFLOW
    assert red(gi, 8, n, out=gi + 16384 - 16) == INVALID            # out over the grads' end
    rsq = lambda grads, fan_in, n, out=_Fake.at(9), ws=_Fake.at(7), wsb=1 << 20, res=_Fake.at(8): \
        lib.reduce_shard_sumsq_interleaved(grads, fan_in, n, 1.0, out, 0, None, 0, ws, wsb, res,
                                           None)
    assert rsq(None, 8, 0) == INVALID
    assert rsq(gi, 65, 0) == UNSUP
    assert rsq(gi + 8, 8, 0) == ALIGN
    assert rsq(gi, 64, 2 ** 59) == OVERFLOW
    assert rsq(gi, 8, n, wsb=0) == CAPACITY
    assert rsq(gi, 8, n, out=gi + 16384 - 16) == INVALID            # out over the grads' end
    assert rsq(gi, 8, n, ws=gi + 8) == INVALID                      # workspace inside the grads
    assert rsq(gi, 8, n, res=gi + 64) == INVALID                    # sum inside the grads


def test_reduce_and_unflatten_validation_errors():
    lib = F.lib()
    g = (ctypes.c_void_p * 2)(_Fake.at(3), _Fake.at(4))
    out = _Fake.at(5)
    assert lib.reduce_shard(g, 2, 0, 1.0, out, None) == OK
    assert lib.reduce_shard(g, 2, 0, 1.0, None, None) == INVALID
    assert lib.reduce_shard(g, 2, 0, 1.0, out + 8, None) == ALIGN
    assert lib.reduce_shard(g, 0, 0, 1.0, out, None) == INVALID
    assert lib.reduce_shard(g, 2, 100, 1.0, _Fake.at(3, 16), None) == INVALID   # overlap
    m = _Fake.at(6)
    assert lib.unflatten_bf16(m, 0, None, 0, out, 0, 0, None) == OK
    assert lib.unflatten_bf16(m + 8, 0, None, 0, out, 0, 0, None) == ALIGN
    assert lib.unflatten_bf16(m, 0, None, 0, out + 1, 0, 0, None) == ALIGN
    assert lib.unflatten_bf16(m, 0, None, 0, None, 0, 0, None) == INVALID
    assert lib.unflatten_bf16(m, 10, None, 0, m + 8, 0, 0, None) == INVALID     # overlap
    assert lib.fsdpshard_stream_copy(m, out, 0, None) == OK
    assert lib.fsdpshard_stream_copy(m, out, 8, None) == INVALID


def test_written_buffers_checked_against_segments_and_inputs():
    """A segment table, gradient input, workspace or sum that overlaps a buffer the call writes is
    refused before anything is launched."""
    lib = F.lib()
    hp = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    a, b, c = _Fake.at(0), _Fake.at(1), _Fake.at(2)
    g = [_Fake.at(3), _Fake.at(4)]
    out = _Fake.at(5)
    n = 100                                   # 400 bytes per fp32 shard, 200 per bf16 one
    # the segment table (n_segments * 32 bytes) inside master, m, v or the bf16 window
    for table in (a + 64, b + 256, c, out + 96):
        assert _step(lib, a, b, c, g, 2, n, table, 2, hp, out, 0, 0) == INVALID
    arr = (ctypes.c_void_p * 2)(*g)
    blk = lib.adamw_shard_step_blocked
    # the blocked state of 100 elements spans 3 * 512 floats
    assert blk(a, arr, 2, n, a + 4096, 1, ctypes.byref(hp), out, 0, 0, None) == INVALID
    clip = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1, 1.0, out + 8)
    assert blk(a, arr, 2, n, None, 0, ctypes.byref(clip), out, 0, 0, None) == INVALID
    f32 = lib.adamw_shard_step_f32grad
    assert f32(a, b, c, g[0], n, b + 32, 1, ctypes.byref(hp), out, 0, 0, None) == INVALID

    ws, res, g32 = _Fake.at(7), _Fake.at(8), _Fake.at(9)
    sq = lib.grad_sumsq_shard
    assert sq(arr, 2, None, n, None, 0, 1.0, g[0] + 32, 8, res, None) == INVALID   # ws in G_0
    assert sq(arr, 2, None, n, None, 0, 1.0, ws, 8, g[1] + 64, None) == INVALID    # sum in G_1
    assert sq(None, 0, g32, n, None, 0, 1.0, g32 + 128, 8, res, None) == INVALID   # ws in grad
    assert sq(None, 0, g32, n, None, 0, 1.0, ws, 8, g32 + 392, None) == INVALID    # sum in grad
    assert sq(arr, 2, None, n, ws, 1, 1.0, ws, 8, res, None) == INVALID            # table = ws
    assert sq(arr, 2, None, n, res - 24, 1, 1.0, ws, 8, res, None) == INVALID      # table over sum

    rs = lib.reduce_shard_sumsq
    o = _Fake.at(10)
    assert rs(arr, 2, n, 1.0, o, 0, None, 0, g[0] + 16, 8, res, None) == INVALID    # ws in G_0
    assert rs(arr, 2, n, 1.0, o, 0, None, 0, ws, 8, g[1], None) == INVALID          # sum in G_1
    assert rs(arr, 2, n, 1.0, o, 0, o + 64, 1, ws, 8, res, None) == INVALID         # table in out
    assert rs(arr, 2, n, 1.0, o, 0, ws, 1, ws, 8, res, None) == INVALID             # table = ws

    m = _Fake.at(6)
    assert lib.unflatten_bf16(m, 10, out + 8, 1, out, 0, 0, None) == INVALID        # table in window


def test_calibration_call_validation():
    lib = F.lib()
    vp = ctypes.c_void_p
    src = (vp * 2)(_Fake.at(1), _Fake.at(2))
    dst = (vp * 1)(_Fake.at(3))
    rw = lambda s_, ns, d_, nd, b, pc=0, sink=None, v=4, t=256, run=0: lib.fsdpshard_stream_rw(
        s_, ns, d_, nd, b, v, t, pc, run, sink, None)
    assert rw(src, 2, dst, 1, 0) == OK
    assert rw(src, 0, dst, 0, 16) == INVALID                        # no stream at all
    assert rw(src, 1, dst, 0, 16) == INVALID                        # pure reads need a sink
    assert rw(src, 9, dst, 1, 16) == INVALID                        # more than 8 streams
    assert rw(src, 2, dst, 1, 8) == INVALID                         # not whole vectors
    assert rw(src, 2, dst, 1, 16, pc=-1) == INVALID
    assert rw(src, 2, dst, 1, 16, run=-1) == INVALID
    assert rw(src, 2, dst, 1, 16, v=3) == UNSUP                     # 1, 2 or 4 vectors
    assert rw(src, 2, dst, 1, 16, v=8) == UNSUP
    assert rw(src, 2, dst, 1, 16, t=128) == UNSUP                   # 256, 512 or 1024 threads
    assert rw((vp * 1)(_Fake.at(1, 8)), 1, dst, 1, 16) == ALIGN
    assert rw(src, 2, (vp * 1)(_Fake.at(1, 16)), 1, 64) == INVALID   # overlap
    assert rw(src, 2, (vp * 2)(_Fake.at(2), _Fake.at(2)), 2, 64) == INVALID  # one array written twice
    assert rw(src, 1, dst, 0, 16, sink=_Fake.at(4, 2)) == ALIGN      # sink not 4-byte aligned
    ph = lambda fi, o, n, g=4, pc=1, run=32, phased=1: lib.fsdpshard_stream_mix_shaped(
        g8, fi, st, o, n, g, pc, run, phased, None)
    g8 = (vp * 8)(*[_Fake.at(10 + r) for r in range(8)])
    st, out = _Fake.at(20), _Fake.at(21)
    assert ph(8, out, 0) == OK
    assert ph(8, out, 0, phased=0) == OK
    gi = _Fake.at(30)
    mi = lambda g, fi, s_, o, n: lib.fsdpshard_stream_mix_interleaved(g, fi, s_, o, n, None)
    assert mi(gi, 8, st, out, 0) == OK
    assert mi(None, 8, st, out, 0) == INVALID
    assert mi(gi, 0, st, out, 0) == INVALID
    assert mi(gi, 65, st, out, 0) == UNSUP
    assert mi(gi, 8, st, out, 12) == INVALID                        # whole vectors only
    assert mi(gi + 8, 8, st, out, 0) == ALIGN
    assert mi(gi, 8, st, gi + 64, 1024) == INVALID                  # out inside the grads
    assert mi(gi, 8, gi + 1024, out, 1024) == INVALID               # state over the grads
    assert ph(2, out, 0) == UNSUP                                   # fan-in 1, 4, 8 only
    assert ph(8, out, 0, g=3) == UNSUP                              # 1, 2 or 4 groups per wave
    assert ph(8, out, 12) == INVALID                                # whole vectors only
    assert ph(8, out, 0, pc=-1) == INVALID
    assert ph(8, out, 0, run=-1) == INVALID
    assert ph(8, out, 0, phased=2) == INVALID
    assert ph(8, _Fake.at(20, 64), 64) == INVALID                   # out inside the state


def test_segment_dtype_matches_struct():
    assert F.SEGMENT_DTYPE.itemsize == ctypes.sizeof(F._Segment) == 32
    assert ctypes.sizeof(F._AdamW) == 72 and ctypes.sizeof(F._Layout) == 48
    L, segs = F.shard_layout([5, 3], 2, 0, 4, [1, 0])
    raw = np.ascontiguousarray(segs).view(np.uint8)
    assert raw.size == 32 * L.n_segments


def test_fp32_grad_step_and_accumulate_validation():
    lib = F.lib()
    hp = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    a, b, c, g, out = (_Fake.at(i) for i in range(5))
    f = lib.adamw_shard_step_f32grad
    assert f(a, b, c, g, 0, None, 0, ctypes.byref(hp), out, 0, 0, None) == OK
    assert f(a, b, c, None, 0, None, 0, ctypes.byref(hp), out, 0, 0, None) == INVALID
    assert f(a, b, c, g + 4, 0, None, 0, ctypes.byref(hp), out, 0, 0, None) == ALIGN
    assert f(a, b, c, a + 64, 100, None, 0, ctypes.byref(hp), out, 0, 0, None) == INVALID  # overlap
    # the bf16 entry point never takes the fp32 path
    arr = (ctypes.c_void_p * 1)(g)
    assert lib.adamw_shard_step(a, b, c, arr, -1, 0, None, 0, ctypes.byref(hp), out, 0, 0, None) == INVALID
    # clipping needs a sum-of-squares pointer, non-negative finite threshold, 8-byte alignment
    clip = F._AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1, 1.0, None)
    assert f(a, b, c, g, 0, None, 0, ctypes.byref(clip), out, 0, 0, None) == INVALID
    clip.grad_sumsq = _Fake.at(6, 4)
    assert f(a, b, c, g, 0, None, 0, ctypes.byref(clip), out, 0, 0, None) == ALIGN
    clip.grad_sumsq = _Fake.at(6)
    assert f(a, b, c, g, 0, None, 0, ctypes.byref(clip), out, 0, 0, None) == OK
    clip.max_grad_norm = -1.0
    assert f(a, b, c, g, 0, None, 0, ctypes.byref(clip), out, 0, 0, None) == INVALID
    acc = lib.reduce_shard_accumulate
    arr2 = (ctypes.c_void_p * 2)(_Fake.at(3), _Fake.at(4))
    assert acc(arr2, 2, 0, 1.0, out, None) == OK
    assert acc(arr2, 2, 0, 1.0, out + 4, None) == ALIGN
    assert acc(arr2, 2, 100, 1.0, _Fake.at(3, 16), None) == INVALID


def test_sumsq_validation_and_workspace():
    lib = F.lib()
    assert F.grad_sumsq_workspace_bytes(0) == 0
    assert F.grad_sumsq_workspace_bytes(1) == 8
    assert F.grad_sumsq_workspace_bytes(32768) == 8          # one partial per 32,768 elements
    assert F.grad_sumsq_workspace_bytes(32769) == 16
    assert F.grad_sumsq_workspace_bytes(905_216_000) == 8 * 27_625
    assert lib.grad_sumsq_workspace_bytes(-1) == -1
    arr = (ctypes.c_void_p * 2)(_Fake.at(3), _Fake.at(4))
    ws, res, g = _Fake.at(7), _Fake.at(8), _Fake.at(9)
    f = lib.grad_sumsq_shard
    assert f(arr, 2, None, 100, None, 0, 1.0, ws, 0, res, None) == CAPACITY
    assert f(arr, 2, None, 100, None, 0, 1.0, None, 8, res, None) == CAPACITY
    assert f(arr, 2, None, 100, None, 0, 1.0, ws, 8, None, None) == INVALID
    assert f(arr, 2, None, 100, None, 0, 1.0, ws, 8, res + 4, None) == ALIGN
    assert f(arr, 2, None, 100, None, 0, 1.0, ws + 4, 8, res, None) == ALIGN
    assert f(None, 0, None, 100, None, 0, 1.0, ws, 8, res, None) == INVALID
    assert f(None, 0, g + 8, 100, None, 0, 1.0, ws, 8, res, None) == ALIGN
    assert f(arr, 2, None, -1, None, 0, 1.0, ws, 8, res, None) == INVALID
    assert f(arr, 2, None, 100, None, 0, 1.0, ws, 8, ws, None) == INVALID          # overlap


def test_noalloc_sumsq_validation():
    # The allocation-free sum of squares takes no workspace and refuses slices longer than its
    # library-owned array covers (CAPACITY), before any HIP call.
    lib = F.lib()
    arr = (ctypes.c_void_p * 2)(_Fake.at(3), _Fake.at(4))
    res = _Fake.at(8)
    f = lib.grad_sumsq_shard_noalloc
    assert F.NOALLOC_MAX_ELEMS == 2 ** 31
    assert f(arr, 2, None, F.NOALLOC_MAX_ELEMS + 1, None, 0, 1.0, res, None) == CAPACITY
    assert f(arr, 2, None, 100, None, 0, 1.0, None, None) == INVALID
    assert f(arr, 2, None, 100, None, 0, 1.0, res + 4, None) == ALIGN
    assert f(arr, 2, None, 100, None, 0, 1.0, _Fake.at(3, 16), None) == INVALID   # sum in G_0
    assert f(arr, 65, None, 100, None, 0, 1.0, res, None) == UNSUP
    assert f(None, 0, None, 100, None, 0, 1.0, res, None) == INVALID


def test_reduce_sumsq_validation():
    # Every error is reported before anything is launched (fake device addresses are never
    # dereferenced).
    lib = F.lib()
    arr = (ctypes.c_void_p * 2)(_Fake.at(3), _Fake.at(4))
    out, ws, res = _Fake.at(10), _Fake.at(7), _Fake.at(8)
    f = lib.reduce_shard_sumsq
    assert f(arr, 2, 100, 1.0, out, 0, None, 0, ws, 0, res, None) == CAPACITY
    assert f(arr, 2, 100, 1.0, out, 0, None, 0, None, 8, res, None) == CAPACITY
    assert f(arr, 2, 100, 1.0, None, 0, None, 0, ws, 8, res, None) == INVALID
    assert f(arr, 2, 100, 1.0, out, 2, None, 0, ws, 8, res, None) == INVALID   # accumulate 0/1
    assert f(arr, 2, 100, 1.0, out, 0, None, 3, ws, 8, res, None) == INVALID   # segs missing
    assert f(arr, 2, 100, 1.0, out, 0, None, 0, ws, 8, None, None) == INVALID
    assert f(arr, 2, 100, 1.0, out + 8, 0, None, 0, ws, 8, res, None) == ALIGN
    assert f(arr, 2, 100, 1.0, out, 0, None, 0, ws, 8, res + 4, None) == ALIGN
    assert f(arr, 2, 100, 1.0, out, 0, None, 0, ws + 4, 8, res, None) == ALIGN
    assert f(arr, 0, 100, 1.0, out, 0, None, 0, ws, 8, res, None) == INVALID
    assert f(arr, 65, 100, 1.0, out, 0, None, 0, ws, 8, res, None) == UNSUP
    assert f(arr, 2, -1, 1.0, out, 0, None, 0, ws, 8, res, None) == INVALID
    assert f(arr, 2, 100, 1.0, out, 0, None, 0, ws, 8, out, None) == INVALID       # overlap
    assert f(arr, 2, 100, 1.0, out, 0, None, 0, out, 8, res, None) == INVALID      # overlap


# ---------------------------------------------------------------------------------- reshard plan

def _execute_plan(pieces, src_shards, dst_len, dtype):
    """Test-side executor of a plan on the host (numpy), to compare with the oracle."""
    out = np.full(dst_len, 99, dtype=dtype)
    for q in pieces:
        a, n_ = int(q["dst_offset"]), int(q["length"])
        if int(q["src_rank"]) < 0:
            out[a:a + n_] = 0
        else:
            s = int(q["src_offset"])
            out[a:a + n_] = src_shards[int(q["src_rank"])][s:s + n_]
    return out


def test_reshard_plan_matches_oracle():
    from oracle import reshard as OR
    rng = random.Random(9)
    for trial in range(300):
        T = rng.randint(0, 8)
        sizes = [rng.choice([0, 1, 2, 5, 16, 17, 33, 100]) for _ in range(T)]
        pa, pb = rng.choice([1, 2, 8, 16]), rng.choice([1, 2, 8, 16])
        na, nb = rng.randint(1, 9), rng.randint(1, 9)
        offs, Pa = OL.flatten_offsets(sizes, pa)
        flat = np.zeros(Pa, dtype=np.float32)
        for o, s in zip(offs, sizes):
            flat[o:o + s] = np.arange(s) + 1000 * o + 0.25
        src = OR.shard(flat, sizes, pa, na)
        want = OR.reshard(src, sizes, pa, pb, nb)
        for k in range(nb):
            pieces = F.reshard_plan(sizes, pa, na, pb, nb, k)
            got = _execute_plan(pieces, src, want[k].size, np.float32)
            assert np.array_equal(got, want[k])
            # pieces tile the shard in order and no two neighbours could have been merged
            pos = 0
            for a, b in zip(pieces, pieces[1:]):
                assert not (a["src_rank"] == b["src_rank"] and
                            (a["src_rank"] < 0 or a["src_offset"] + a["length"] == b["src_offset"]))
            for q in pieces:
                assert q["dst_offset"] == pos and q["length"] > 0
                pos += int(q["length"])
            assert pos == want[k].size


def test_reshard_plan_same_layout_is_one_piece_per_source_overlap():
    sizes = [1000, 7, 2000]
    for k in range(4):
        pieces = F.reshard_plan(sizes, 1, 4, 1, 4, k)
        assert len(pieces) == 1 and pieces[0]["src_rank"] == k and pieces[0]["src_offset"] == 0


def test_reshard_plan_errors_and_capacity():
    lib = F.lib()
    sizes = (ctypes.c_int64 * 3)(5, 6, 7)
    n = ctypes.c_int32(0)
    assert lib.reshard_plan(sizes, 3, 4, 2, 1, 3, 0, None, 0, ctypes.byref(n)) == OK and n.value > 1
    buf = (F._Piece * 1)()
    assert lib.reshard_plan(sizes, 3, 4, 2, 1, 3, 0, buf, 1, ctypes.byref(n)) == CAPACITY
    assert lib.reshard_plan(sizes, 3, 0, 2, 1, 3, 0, None, 0, ctypes.byref(n)) == INVALID
    assert lib.reshard_plan(sizes, 3, 4, 2, 1, 3, 3, None, 0, ctypes.byref(n)) == INVALID
    assert lib.reshard_plan(sizes, 3, 4, 0, 1, 3, 0, None, 0, ctypes.byref(n)) == INVALID
    assert lib.reshard_plan(sizes, 3, 4, 2, 1, 3, 0, None, 0, None) == INVALID


def test_reshard_copy_validation():
    lib = F.lib()
    src = (ctypes.c_void_p * 2)(_Fake.at(1), _Fake.at(2))
    elems = (ctypes.c_int64 * 2)(100, 100)
    P = F._Piece
    good = (P * 2)(P(0, 0, 50, 0, 0), P(0, 50, 50, 1, 0))
    d = _Fake.at(3)
    assert lib.reshard_copy(src, elems, 2, d, 100, good, 0, 4, None) == OK
    bad_rank = (P * 1)(P(0, 0, 10, 2, 0))
    assert lib.reshard_copy(src, elems, 2, d, 100, bad_rank, 1, 4, None) == INVALID
    oob = (P * 1)(P(95, 0, 10, 0, 0))
    assert lib.reshard_copy(src, elems, 2, d, 100, oob, 1, 4, None) == INVALID
    oob_dst = (P * 1)(P(0, 95, 10, 0, 0))
    assert lib.reshard_copy(src, elems, 2, d, 100, oob_dst, 1, 4, None) == INVALID
    overlap = (P * 2)(P(0, 10, 20, 0, 0), P(0, 0, 15, 1, 0))
    assert lib.reshard_copy(src, elems, 2, d, 100, overlap, 2, 4, None) == INVALID
    assert lib.reshard_copy(src, elems, 2, d + 2, 100, good, 0, 4, None) == ALIGN
    assert lib.reshard_copy(src, elems, 2, d, 100, good, 0, 3, None) == INVALID
    assert lib.reshard_copy(src, elems, 2, _Fake.at(1, 16), 100, good, 0, 4, None) == INVALID
    # an empty destination shard may be NULL; a non-empty one may not
    assert lib.reshard_copy(src, elems, 2, None, 0, good, 0, 4, None) == OK
    assert lib.reshard_copy(src, elems, 2, None, 100, good, 0, 4, None) == INVALID
    assert lib.reshard_copy(src, elems, 2, None, 0, good, 1, 4, None) == INVALID


def test_binding_checks_buffer_sizes_before_any_call():
    # The library sees only pointers; the binding rejects buffers too small for the call (these
    # checks run before any device pointer is taken, so CPU tensors exercise them).
    import torch
    with pytest.raises(ValueError, match="segs holds 31 bytes, 32 needed"):
        F._segs(torch.zeros(31, dtype=torch.uint8), 1)
    F._segs(None, 0)
    with pytest.raises(ValueError, match="dst holds 8 bytes, 16 needed"):
        F.stream_copy(torch.zeros(4, dtype=torch.float32), torch.zeros(2, dtype=torch.float32))
    with pytest.raises(ValueError, match="one element size"):
        F.reshard_copy([torch.zeros(4, dtype=torch.float32)], torch.zeros(4, dtype=torch.int16),
                       np.zeros(0, dtype=F.PIECE_DTYPE))
