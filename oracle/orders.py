"""Scan orders over a 2-D feature map, and the scan along them (fp64 oracle).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the HIP path never does.

A [height, width] map is flattened row-major, token t = r * width + c (Mamba in the
YOLO26 backbone page, section 1.2: the image is flattened into a sequence and
scanned by rows, by columns, or crosswise in several directions; section 2.2: the
row scan forward and backward, added elementwise; section 4.4: four directions,
rows and columns both ways).  A scan order is the sequence of tokens a direction
visits; the output of every direction lands at the tokens' own positions, the
directions are summed, and the gate is applied once.

The spiral is the Samba page's order (section 3.1): start at the image centre and
wind outwards clockwise, each step to an unvisited neighbour -- read here as the
square spiral right 1, down 1, left 2, up 2, right 3, ... (rows grow downwards, so
this turns clockwise on screen), skipping positions outside the map; the centre of
an even side is the lower of its two middle indices.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle

ROW, ROW_REV, COL, COL_REV, INDEX, INDEX_REV = range(6)


def row_order(h: int, w: int) -> np.ndarray:
    return np.arange(h * w, dtype=np.int64)


def col_order(h: int, w: int) -> np.ndarray:
    """Column by column, top to bottom: token (r, c) visited at step c * h + r."""
    out = np.empty(h * w, dtype=np.int64)
    k = 0
    for c in range(w):
        for r in range(h):
            out[k] = r * w + c
            k += 1
    return out


def spiral_order(h: int, w: int) -> np.ndarray:
    """Centre-out clockwise square spiral over an h x w map (row-major tokens)."""
    r, c = (h - 1) // 2, (w - 1) // 2
    out = [r * w + c]
    moves = [(0, 1), (1, 0), (0, -1), (-1, 0)]  # right, down, left, up
    run, m = 1, 0
    while len(out) < h * w:
        for _ in range(2):  # two legs per run length
            dr, dc = moves[m % 4]
            for _ in range(run):
                r, c = r + dr, c + dc
                if 0 <= r < h and 0 <= c < w:
                    out.append(r * w + c)
            m += 1
        run += 1
    return np.asarray(out, dtype=np.int64)


def visit_order(kind: int, h: int, w: int, index=None) -> np.ndarray:
    if kind in (ROW, ROW_REV):
        o = row_order(h, w)
    elif kind in (COL, COL_REV):
        o = col_order(h, w)
    else:
        o = np.asarray(index, dtype=np.int64)
    return o[::-1].copy() if kind in (ROW_REV, COL_REV, INDEX_REV) else o


def scan_multi(u, z, dirs, kinds, h, w, index=None, softplus=True, nthreads=1):
    """out = (sum over directions k of the scan visiting tokens in order k) * silu(z).
    dirs[k] has delta, A, B, C and optional D, delta_bias, all in token-position
    layout; each direction's inputs are gathered into its visiting order, scanned
    forward, and its output put back at the tokens' positions."""
    u = np.asarray(u, np.float64)
    b, d, L = u.shape
    if L != h * w:
        raise ValueError("len must be height * width")
    total = np.zeros((b, d, L))
    for p, kind in zip(dirs, kinds):
        o = visit_order(kind, h, w, index)
        g = lambda a: np.ascontiguousarray(np.asarray(a, np.float64)[..., o])
        y = oracle.sscan_fwd(g(u), g(p["delta"]), p["A"], g(p["B"]), g(p["C"]), p.get("D"), None,
                             p.get("delta_bias"), softplus=softplus, nthreads=nthreads)
        total[..., o] += y
    if z is not None:
        zz = np.asarray(z, np.float64)
        total = total * (zz / (1.0 + np.exp(-zz)))
    return total


def scan_multi_bwd(u, z, g, dirs, kinds, h, w, index=None, softplus=True, nthreads=1):
    """Gradients of sum(g * scan_multi(u, z, dirs, kinds, h, w, index)) (fp64).

    The chain rule through the sum and the gate: with s the sum of the directions'
    outputs, out = s * silu(z), so ds = g * silu(z) reaches every direction's output
    and dz = g * s * silu'(z).  Each direction's gradients are the one-direction
    backward (oracle.sscan_bwd, no gate) of its inputs gathered into its visiting
    order, with ds gathered the same way; they are put back at the tokens'
    positions (the gather's transpose: a permutation, so position o[i] receives
    visit step i).  du sums over the directions; the parameter gradients are per
    direction.  ``index`` must be a permutation of the tokens.  Returns
    {"du", "dz" (None without z), "dirs": [{ddelta, ddelta_bias, dA, dB, dC, dD}]}."""
    u = np.asarray(u, np.float64)
    b, d, L = u.shape
    if L != h * w:
        raise ValueError("len must be height * width")
    g = np.asarray(g, np.float64)
    dz = None
    if z is not None:
        zz = np.asarray(z, np.float64)
        sig = 1.0 / (1.0 + np.exp(-zz))
        s = scan_multi(u, None, dirs, kinds, h, w, index, softplus=softplus, nthreads=nthreads)
        dz = g * s * (sig * (1.0 + zz * (1.0 - sig)))
        ds = g * (zz * sig)
    else:
        ds = g
    du = np.zeros((b, d, L))
    grads = []
    for p, kind in zip(dirs, kinds):
        o = visit_order(kind, h, w, index)
        if not np.array_equal(np.sort(o), np.arange(L)):
            raise ValueError("the index order must be a permutation of the tokens")
        gat = lambda a: np.ascontiguousarray(np.asarray(a, np.float64)[..., o])
        q = dict(delta=gat(p["delta"]), A=p["A"], B=gat(p["B"]), C=gat(p["C"]), D=p.get("D"),
                 delta_bias=p.get("delta_bias"))
        r = oracle.sscan_bwd(gat(u), None, gat(ds), [q], softplus=softplus, nthreads=nthreads)
        du[..., o] += r["du"]
        gd = r["dirs"][0]
        out = dict(gd)
        for name in ("ddelta", "dB", "dC"):
            back = np.empty_like(gd[name])
            back[..., o] = gd[name]
            out[name] = back
        grads.append(out)
    return {"du": du, "dz": dz, "dirs": grads}
