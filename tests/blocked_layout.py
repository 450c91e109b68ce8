"""The blocked placement of a slice's optimizer state, written out for the tests.

This is a placement of the state in memory, not part of the method: the values and their
positions in the slice are those of the three separate shards ("FSDP: Fully Sharded Data Parallel
Training at Scale", sharding a linear layer: grad, m and v cover the same positions).  Element i
of the slice, in block b = i // STATE_BLOCK at offset o = i % STATE_BLOCK, keeps its master at
3*b*STATE_BLOCK + o, its m at (3*b + 1)*STATE_BLOCK + o and its v at (3*b + 2)*STATE_BLOCK + o of
one array.  The tests use it to lay out inputs for the blocked-state entry points and to read
their results back; the oracle's arithmetic runs on the separate arrays.

The interleaved placement of a slice's F gradient contributions is the same idea for the inputs
of the reduce-scatter ("FSDP: Fully Sharded Data Parallel Training at Scale", communication
pattern of one unit): block b of one array holds every contribution's elements
[b*STATE_BLOCK, (b+1)*STATE_BLOCK) one contribution after another, so contribution r's element i
sits at (b*F + r)*STATE_BLOCK + o.
"""

import numpy as np

STATE_BLOCK = 512


def blocked_state_len(n):
    return 3 * (-(-n // STATE_BLOCK)) * STATE_BLOCK


def to_blocked(master, m, v, fill=0.0):
    """The blocked array of a slice (positions past n in the last block hold `fill`)."""
    n = len(master)
    out = np.full(blocked_state_len(n), fill, dtype=np.float32)
    for i in range(0, n, STATE_BLOCK):
        b, k = i // STATE_BLOCK, min(STATE_BLOCK, n - i)
        for s, arr in enumerate((master, m, v)):
            start = (3 * b + s) * STATE_BLOCK
            out[start:start + k] = arr[i:i + k]
    return out


def from_blocked(state, n):
    """(master, m, v) of an n-element slice from its blocked array."""
    parts = [np.empty(n, dtype=np.float32) for _ in range(3)]
    for i in range(0, n, STATE_BLOCK):
        b, k = i // STATE_BLOCK, min(STATE_BLOCK, n - i)
        for s in range(3):
            start = (3 * b + s) * STATE_BLOCK
            parts[s][i:i + k] = state[start:start + k]
    return tuple(parts)


def interleaved_len(fan_in, n):
    return fan_in * (-(-n // STATE_BLOCK)) * STATE_BLOCK


def to_interleaved(contribs, fill=0):
    """The interleaved array of F contributions of equal length n (positions past n in the last
    block hold `fill`)."""
    F = len(contribs)
    n = len(contribs[0])
    out = np.full(interleaved_len(F, n), fill, dtype=np.uint16)
    for i in range(0, n, STATE_BLOCK):
        b, k = i // STATE_BLOCK, min(STATE_BLOCK, n - i)
        for r, c in enumerate(contribs):
            start = (b * F + r) * STATE_BLOCK
            out[start:start + k] = c[i:i + k]
    return out
