"""The fused step driven from plain C (tests/c_abi/gpu_step.c: hipMalloc, shard_layout,
adamw_shard_step on the null stream, no Python in the call path), checked against the oracle.

The test writes seeded inputs to a file, runs the program as a child process and compares its
output with the oracle's steps (fp32 state within relative 1e-5, bf16 within 1 ulp), and checks
that the guard elements around the slice's bf16 window are untouched.
"""

import os
import subprocess
import tempfile

import numpy as np
import pytest

import workloads as W
from oracle import layout as OL
from oracle import step as OS
from gpu_helpers import assert_bf16, assert_f32, say

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "bin", "gpu_step")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, grad_scale=0.5)


@pytest.mark.parametrize("sizes,pad,N,k,F_in,S", [
    ([70001, 5, 12000, 1, 333], 16, 3, 1, 4, 3),
    ([1_000_003], 1, 8, 3, 8, 2),
    ([257, 4099, 16, 65536 + 3], 8, 2, 0, 1, 2),
])
def test_c_driven_step_matches_oracle(sizes, pad, N, k, F_in, S):
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: run `python tests/c_abi/build.py` (build() does)")
    wd = [i % 2 == 0 for i in range(len(sizes))]
    lo, hi, segs = OL.segments(sizes, pad, [int(x) for x in wd], N, k)
    n = hi - lo
    flags = np.zeros(n, dtype=np.int64)
    for s in segs:
        flags[s["shard_begin"]: s["shard_begin"] + s["length"]] = s["flags"]
    say(f"C-driven step: n={n} lo={lo} F={F_in} steps={S}")
    master = W.np_f32_uniform([70, n], n, -0.05, 0.05)
    m = W.np_f32_normal([71, n], n, 1e-3)
    v = np.abs(W.np_f32_normal([72, n], n, 1e-6)).astype(np.float32)
    grads = [W.np_bf16_normal([73, r], n, 1e-2) for r in range(F_in)]
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(b"FSDPIN1\0")
            f.write(np.array([len(sizes), pad, N, k, F_in, S], dtype=np.int64).tobytes())
            f.write(np.array([HP[x] for x in ("lr", "beta1", "beta2", "eps", "weight_decay",
                                              "grad_scale")], dtype=np.float64).tobytes())
            f.write(np.array(sizes, dtype=np.int64).tobytes())
            f.write(np.array(wd, dtype=np.uint8).tobytes())
            for a in (master, m, v):
                f.write(a.astype(np.float32).tobytes())
            for g in grads:
                f.write(g.astype(np.uint16).tobytes())
        run = subprocess.run([BIN, fin, fout], capture_output=True, text=True, timeout=120)
        assert run.returncode == 0, run.stderr
        say("  " + run.stdout.strip())
        raw = open(fout, "rb").read()
    hdr = np.frombuffer(raw[:24], dtype=np.int64)
    assert (int(hdr[0]), int(hdr[1])) == (n, lo)
    phase = int(hdr[2])
    st = np.frombuffer(raw[24:24 + 12 * n], dtype=np.float32).reshape(3, n)
    window = np.frombuffer(raw[24 + 12 * n:], dtype=np.uint16)
    assert window.size == n + phase + 16

    wm, wmm, wv = master.copy(), m.copy(), v.copy()
    for t in range(1, S + 1):
        wm, wmm, wv, out = OS.shard_step(wm, wmm, wv, grads, flags, HP, t)
    assert_f32(st[0], wm, "master")
    assert_f32(st[1], wmm, "m")
    assert_f32(st[2], wv, "v")
    assert_bf16(window[8 + phase: 8 + phase + n], out, "flat")
    assert (window[:8 + phase] == 0xABCD).all() and (window[8 + phase + n:] == 0xABCD).all()
