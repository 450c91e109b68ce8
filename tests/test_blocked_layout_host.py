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


def test_interleaved_gradient_layout_by_hand():
    # Three contributions of 515 elements: block 0 holds elements 0..511 of contribution 0, then
    # of 1, then of 2; block 1 holds elements 512..514 of each at the starts of its three slots.
    n = 515
    c = [np.arange(n, dtype=np.uint16) + 1000 * r for r in range(3)]
    g = BL.to_interleaved(c, fill=0xFFFF)
    assert g.size == BL.interleaved_len(3, n) == 6 * 512
    assert g[0] == 0 and g[511] == 511
    assert g[512] == 1000 and g[1023] == 1511
    assert g[1024] == 2000 and g[1535] == 2511
    assert list(g[1536:1539]) == [512, 513, 514] and g[1539] == 0xFFFF
    assert list(g[2048:2051]) == [1512, 1513, 1514] and g[2051] == 0xFFFF
    assert list(g[2560:2563]) == [2512, 2513, 2514] and (g[2563:] == 0xFFFF).all()


def test_interleaved_gradient_positions():
    rng = np.random.default_rng(4)
    for F in (1, 2, 5, 8):
        for n in (1, 511, 512, 513, 1500, 4099):
            c = [rng.integers(0, 1 << 16, n, dtype=np.uint16) for _ in range(F)]
            g = BL.to_interleaved(c)
            assert g.size == F * -(-n // 512) * 512
            if F == 1:   # one contribution: the interleaved array is the contribution itself
                assert np.array_equal(g[:n], c[0])
            for i in (0, n - 1, n // 2):
                blk, o = divmod(i, BL.STATE_BLOCK)
                for r in range(F):
                    assert g[(blk * F + r) * BL.STATE_BLOCK + o] == c[r][i]
