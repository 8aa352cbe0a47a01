"""Pins of the 2-D scan orders and the multi-order scan (oracle/orders.py).

No HIP code is involved.
"""
import math

import numpy as np
import pytest

from oracle import oracle, orders


def _params(rng, b, d, L):
    return dict(delta=rng.normal(0.0, 0.5, (b, d, L)), A=-np.exp(rng.uniform(-1.0, 1.0, (d, 16))),
                B=rng.normal(size=(b, 16, L)), C=rng.normal(size=(b, 16, L)), D=rng.normal(size=d),
                delta_bias=rng.uniform(-3.0, 0.0, d))


def test_column_order_is_the_transposed_map():
    """Scanning by columns = transposing the map (numpy) and scanning by rows:
    catches a swapped height/width or a row-major column index."""
    rng = np.random.default_rng(1)
    b, d, h, w = 2, 3, 5, 7
    L = h * w
    u, z = rng.normal(size=(b, d, L)), rng.normal(size=(b, d, L))
    p = _params(rng, b, d, L)
    got = orders.scan_multi(u, z, [p], [orders.COL], h, w)
    T = lambda a: np.ascontiguousarray(a.reshape(a.shape[:-1] + (h, w)).swapaxes(-1, -2).reshape(a.shape))
    yT = oracle.sscan_fwd(T(u), T(p["delta"]), p["A"], T(p["B"]), T(p["C"]), p["D"], T(z), p["delta_bias"])
    back = yT.reshape(b, d, w, h).swapaxes(-1, -2).reshape(b, d, L)
    np.testing.assert_allclose(got, back, rtol=1e-13, atol=1e-13)


def test_row_orders_are_the_plain_scans_and_sum_before_gate():
    """Row forward + row reverse = the bidirectional scan (YOLO26 page section 2.2:
    the two row directions added elementwise, the gate once)."""
    rng = np.random.default_rng(2)
    b, d, h, w = 2, 2, 3, 6
    L = h * w
    u, z = rng.normal(size=(b, d, L)), rng.normal(size=(b, d, L))
    pf, pr = _params(rng, b, d, L), _params(rng, b, d, L)
    got = orders.scan_multi(u, z, [pf, pr], [orders.ROW, orders.ROW_REV], h, w)
    np.testing.assert_allclose(got, oracle.sscan_bidir(u, z, pf, pr), rtol=1e-13, atol=1e-13)
    single = orders.scan_multi(u, None, [pf], [orders.ROW], h, w)
    np.testing.assert_allclose(single, oracle.sscan_fwd(u, pf["delta"], pf["A"], pf["B"], pf["C"], pf["D"], None,
                                                        pf["delta_bias"]), rtol=1e-13, atol=1e-13)


def test_reversed_index_order_and_permutation_equivariance():
    """A scan along any order equals the row scan of the map whose tokens were
    permuted into that order; the reversed order is the reverse scan of it."""
    rng = np.random.default_rng(3)
    b, d, h, w = 1, 2, 4, 4
    L = h * w
    perm = rng.permutation(L)
    u = rng.normal(size=(b, d, L))
    p = _params(rng, b, d, L)
    g = lambda a: np.ascontiguousarray(a[..., perm])
    for kind, rev in ((orders.INDEX, False), (orders.INDEX_REV, True)):
        got = orders.scan_multi(u, None, [p], [kind], h, w, index=perm)
        y = oracle.sscan_fwd(g(u), g(p["delta"]), p["A"], g(p["B"]), g(p["C"]), p["D"], None, p["delta_bias"],
                             reverse=rev)
        ref = np.empty_like(y)
        ref[..., perm] = y
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("h,w", [(1, 1), (1, 6), (5, 5), (4, 4), (3, 8), (7, 2), (9, 9)])
def test_spiral_is_a_permutation_starting_at_the_centre(h, w):
    o = orders.spiral_order(h, w)
    assert sorted(o.tolist()) == list(range(h * w))
    assert o[0] == ((h - 1) // 2) * w + (w - 1) // 2


@pytest.mark.parametrize("n", [3, 5, 9, 13])
def test_spiral_on_odd_squares_matches_ring_and_angle_sort(n):
    """Independent construction for odd squares: visit rings by Chebyshev distance
    from the centre; within ring k start just below the top-right corner
    (row offset 1 - k, column offset k) and go clockwise, i.e. sort by the
    clockwise angle from that start (atan2 with rows growing downwards).  Every
    step moves to one of the 8 neighbours."""
    o = orders.spiral_order(n, n)
    c = (n - 1) // 2
    cells = []
    for r in range(n):
        for col in range(n):
            dr, dc = r - c, col - c
            k = max(abs(dr), abs(dc))
            if k == 0:
                key = (0, 0.0)
            else:
                start = math.atan2(1 - k, k)  # angle of the ring's first cell (x = col, y = row)
                ang = (math.atan2(dr, dc) - start) % (2 * math.pi)
                key = (k, ang)
            cells.append((key, r * n + col))
    ref = [t for _, t in sorted(cells)]
    assert o.tolist() == ref
    rc = [(t // n, t % n) for t in o]
    assert all(max(abs(a[0] - b[0]), abs(a[1] - b[1])) == 1 for a, b in zip(rc, rc[1:]))


def test_clockwise_first_moves():
    """Rows grow downwards: right, then down, then left is a clockwise turn."""
    o = orders.spiral_order(5, 5)
    rc = [(t // 5, t % 5) for t in o[:4]]
    assert rc == [(2, 2), (2, 3), (3, 3), (3, 2)]
