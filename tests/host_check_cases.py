"""Random cases for tests/c_abi/host_check (the host entry points called from plain C), checked
against the oracle.  Shared by the test of the regular build (linked against libfsdpshard.so) and
the test of the sanitized build (the host layout source compiled with AddressSanitizer and UBSan).

The layout and segment table must equal the oracle's; the reshard plan is applied to the oracle's
source shards with NumPy and must rebuild the oracle's destination shard.
"""

import random
import subprocess

import numpy as np

from oracle import layout as OL
from oracle import reshard as OR


def run(binary, sizes, wd, pad, N, k, pad2, N2, k2, env=None):
    text = f"{len(sizes)} {pad} {N} {k} {pad2} {N2} {k2}\n"
    text += " ".join(map(str, sizes)) + "\n" + " ".join(str(int(x)) for x in wd) + "\n"
    out = subprocess.run([binary], input=text, capture_output=True, text=True, timeout=60, env=env)
    assert out.returncode == 0, out.stderr
    assert out.stderr == "", out.stderr
    lines = [ln.split() for ln in out.stdout.splitlines()]
    rec = {"segs": [], "pieces": []}
    for ln in lines:
        if ln[0] == "abi":
            rec["abi"] = int(ln[1])
        elif ln[0] == "layout":
            rec["layout"] = list(map(int, ln[1:]))
        elif ln[0] == "seg":
            rec["segs"].append(tuple(map(int, ln[1:])))
        elif ln[0] == "plan":
            rec["count"] = int(ln[1])
        elif ln[0] == "piece":
            rec["pieces"].append(tuple(map(int, ln[1:])))
        elif ln[0] == "badrank":
            rec["badrank"] = (int(ln[1]), " ".join(ln[2:]))
    return rec


def check_random_cases(binary, seed=5, trials=60, env=None):
    rng = random.Random(seed)
    for trial in range(trials):
        T = rng.randint(1, 12)
        sizes = [rng.choice([0, 1, 3, 8, 17, 100, 1001, 4096]) for _ in range(T)]
        wd = [rng.random() < 0.5 for _ in range(T)]
        pad, pad2 = rng.choice([1, 2, 8, 16]), rng.choice([1, 4, 16])
        N, N2 = rng.randint(1, 9), rng.randint(1, 9)
        k, k2 = rng.randrange(N), rng.randrange(N2)
        rec = run(binary, sizes, wd, pad, N, k, pad2, N2, k2, env=env)
        assert rec["abi"] == 1

        lo, hi, segs = OL.segments(sizes, pad, [int(x) for x in wd], N, k)
        offs, P = OL.flatten_offsets(sizes, pad)
        real = sum(s["length"] for s in segs if not s["flags"] & OL.PADDING)
        tensors = len({s["tensor_id"] for s in segs})
        assert rec["layout"] == [P, lo, hi, hi - lo, real, len(segs), tensors], (trial, sizes)
        assert rec["segs"] == [(s["shard_begin"], s["length"], s["tensor_offset"], s["tensor_id"],
                                s["flags"]) for s in segs]

        # Apply the plan to the oracle's shards: it must rebuild the oracle's destination shard.
        flat = np.zeros(P, dtype=np.int64)
        for i, (o, s) in enumerate(zip(offs, sizes)):
            flat[o:o + s] = 1 + 1000 * i + np.arange(s)
        src = OR.shard(flat, sizes, pad, N)
        want = OR.reshard(src, sizes, pad, pad2, N2)[k2]
        got = np.full(want.size, -1, dtype=np.int64)
        assert rec["count"] == len(rec["pieces"])
        for r, so, do, ln in rec["pieces"]:
            assert (got[do:do + ln] == -1).all()                        # pieces are disjoint
            got[do:do + ln] = 0 if r < 0 else src[r][so:so + ln]
        assert np.array_equal(got, want), (trial, sizes, pad, N, pad2, N2, k2)
        assert rec["badrank"] == (1, "invalid argument")
