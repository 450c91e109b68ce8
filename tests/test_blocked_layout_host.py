"""The tests' blocked-state placement (tests/blocked_layout.py), checked by hand and by round
trips, so the blocked-state GPU tests lay out and read back what the header defines."""

import numpy as np

import blocked_layout as BL


def test_blocked_state_layout_by_hand():
    # Slice of 515 elements: block 0 holds elements 0..511 of master, then of m, then of v;
    # block 1 holds elements 512..514 of each, at the starts of its three 512-slots.
    n = 515
    master = np.arange(n, dtype=np.float32)
    m = master + 1000.0
    v = master + 2000.0
    st = BL.to_blocked(master, m, v, fill=-1.0)
    assert st.size == BL.blocked_state_len(n) == 6 * 512
    assert st[0] == 0.0 and st[511] == 511.0
    assert st[512] == 1000.0 and st[1023] == 1511.0
    assert st[1024] == 2000.0 and st[1535] == 2511.0
    assert list(st[1536:1539]) == [512.0, 513.0, 514.0] and st[1539] == -1.0
    assert list(st[2048:2051]) == [1512.0, 1513.0, 1514.0] and st[2051] == -1.0
    assert list(st[2560:2563]) == [2512.0, 2513.0, 2514.0] and (st[2563:] == -1.0).all()


def test_blocked_state_round_trip_and_element_positions():
    rng = np.random.default_rng(3)
    for n in (0, 1, 7, 511, 512, 513, 1024, 1500, 4099):
        a, b, c = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
        st = BL.to_blocked(a, b, c)
        back = BL.from_blocked(st, n)
        assert all(np.array_equal(x, y) for x, y in zip(back, (a, b, c)))
        for i in ([0, n - 1, n // 2] if n else []):
            blk, o = divmod(i, BL.STATE_BLOCK)
            for s, arr in enumerate((a, b, c)):
                assert st[(3 * blk + s) * BL.STATE_BLOCK + o] == arr[i]
