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


# --- backward along several orders ---------------------------------------------------------------

def _torch_multi(u, z, dirs, kinds, h, w, index, softplus=True):
    """The forward definition in fp64 torch ops: every direction walks its visiting
    order token by token (its own recurrence, no gathered copies), writes each
    output at the token it visits, the outputs are summed and gated."""
    import torch
    b, d, L = u.shape
    total = torch.zeros_like(u)
    for p, kind in zip(dirs, kinds):
        if kind in (orders.ROW, orders.ROW_REV):
            steps = [t for t in range(L)]
        elif kind in (orders.COL, orders.COL_REV):
            steps = [r * w + c for c in range(w) for r in range(h)]
        else:
            steps = [int(t) for t in index]
        if kind % 2 == 1:
            steps = steps[::-1]
        x = p["delta"] + p["delta_bias"][None, :, None]
        dt = torch.nn.functional.softplus(x) if softplus else x
        hs = torch.zeros(b, d, p["A"].shape[1], dtype=torch.float64)
        cols = [None] * L
        for t in steps:
            hs = torch.exp(dt[:, :, t, None] * p["A"][None]) * hs + (dt[:, :, t] * u[:, :, t])[..., None] * \
                p["B"][:, None, :, t]
            cols[t] = (hs * p["C"][:, None, :, t]).sum(-1) + p["D"][None] * u[:, :, t]
        total = total + torch.stack(cols, -1)
    return total * torch.nn.functional.silu(z) if z is not None else total


@pytest.mark.parametrize("kinds,gate", [
    ((orders.ROW, orders.ROW_REV, orders.COL, orders.COL_REV, orders.INDEX, orders.INDEX_REV), True),
    ((orders.COL, orders.INDEX_REV), False),
    ((orders.COL_REV,), True),
])
def test_multi_bwd_matches_autograd(kinds, gate):
    """Every gradient of the multi-order backward against PyTorch's reverse-mode
    differentiation of the token-by-token definition above (a library routine that
    shares nothing with the gather/put-back of the oracle): a wrong put-back index,
    a transposed column order or a gate applied per direction fails here."""
    import torch
    rng = np.random.default_rng(50 + len(kinds))
    b, d, h, w = 2, 3, 3, 5
    L = h * w
    perm = np.asarray(orders.spiral_order(h, w))
    u, z, g = (rng.normal(size=(b, d, L)) for _ in range(3))
    dirs = [_params(rng, b, d, L) for _ in kinds]
    got = orders.scan_multi_bwd(u, z if gate else None, g, dirs, list(kinds), h, w, index=perm)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    ut, zt = T(u), T(z)
    dts = [{k: T(v) for k, v in p.items()} for p in dirs]
    out = _torch_multi(ut, zt if gate else None, dts, kinds, h, w, perm)
    (out * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(got["du"], ut.grad.numpy(), rtol=1e-10, atol=1e-12)
    if gate:
        np.testing.assert_allclose(got["dz"], zt.grad.numpy(), rtol=1e-10, atol=1e-12)
    else:
        assert got["dz"] is None
    keys = {"ddelta": "delta", "ddelta_bias": "delta_bias", "dA": "A", "dB": "B", "dC": "C", "dD": "D"}
    for k in range(len(kinds)):
        for gname, pname in keys.items():
            ref = dts[k][pname].grad.numpy()
            np.testing.assert_allclose(got["dirs"][k][gname], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max(),
                                       err_msg=f"dir{k}.{gname}")


def test_multi_bwd_matches_central_differences():
    """A sample of entries against central differences of the forward oracle
    scan_multi (pinned above), four directions with a gate."""
    rng = np.random.default_rng(61)
    b, d, h, w = 1, 2, 4, 3
    L = h * w
    kinds = [orders.ROW_REV, orders.COL, orders.INDEX, orders.INDEX_REV]
    perm = rng.permutation(L)
    u, z, g = (rng.normal(size=(b, d, L)) for _ in range(3))
    dirs = [_params(rng, b, d, L) for _ in kinds]
    got = orders.scan_multi_bwd(u, z, g, dirs, kinds, h, w, index=perm)
    loss = lambda uu, zz, dd: float(np.sum(g * orders.scan_multi(uu, zz, dd, kinds, h, w, index=perm)))
    e = 1e-5
    for idx in ((0, 0, 0), (0, 1, 7), (0, 1, 11)):
        for name, arr in (("du", u), ("dz", z)):
            hi, lo = arr.copy(), arr.copy()
            hi[idx] += e
            lo[idx] -= e
            args = lambda a: (a, z, dirs) if name == "du" else (u, a, dirs)
            ref = (loss(*args(hi)) - loss(*args(lo))) / (2 * e)
            assert abs(got[name][idx] - ref) <= 1e-6 * (1 + abs(ref)), (name, idx)
    for k in range(len(kinds)):
        for gname, pname, idx in (("ddelta", "delta", (0, 1, 5)), ("dB", "B", (0, 3, 9)), ("dC", "C", (0, 15, 2)),
                                  ("dA", "A", (1, 4)), ("dD", "D", (0,)), ("ddelta_bias", "delta_bias", (1,))):
            def mut(sign, k=k, pname=pname, idx=idx):
                nd = [dict(p) for p in dirs]
                arr = nd[k][pname].copy()
                arr[idx] += sign * e
                nd[k][pname] = arr
                return loss(u, z, nd)
            ref = (mut(1) - mut(-1)) / (2 * e)
            assert abs(got["dirs"][k][gname][idx] - ref) <= 1e-6 * (1 + abs(ref)), (k, gname, idx)


def test_multi_bwd_rows_are_the_bidirectional_backward():
    """Rows forward + reverse: the gated bidirectional backward of the C oracle."""
    rng = np.random.default_rng(62)
    b, d, h, w = 2, 2, 3, 4
    L = h * w
    u, z, g = (rng.normal(size=(b, d, L)) for _ in range(3))
    dirs = [_params(rng, b, d, L) for _ in range(2)]
    got = orders.scan_multi_bwd(u, z, g, dirs, [orders.ROW, orders.ROW_REV], h, w)
    ref = oracle.sscan_bwd(u, z, g, dirs)
    for name in ("du", "dz"):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-12, atol=1e-13)
    for k in range(2):
        for gname in ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD"):
            np.testing.assert_allclose(got["dirs"][k][gname], ref["dirs"][k][gname], rtol=1e-12, atol=1e-12)
