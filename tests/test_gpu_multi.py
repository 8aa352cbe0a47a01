"""GPU parity of the multi-order scan of a 2-D map (``sscan_multi``) against the
fp64 oracle of the visiting orders (oracle/orders.py, pinned in
test_oracle_orders_pins.py).
"""
import os
import zlib

import numpy as np
import pytest
import torch

from oracle import oracle, orders
from parity import TOL, metrics
from selective_state_space_sscan_amd import inputs as I
from selective_state_space_sscan_amd import sscan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NTHREADS = min(16, oracle.default_threads())


@pytest.fixture(scope="module", autouse=True)
def _lib():
    sscan.load_library()  # raises if the extension is missing: no fallback
    if not os.path.exists(oracle.LIB):
        oracle.build(force=True)


def draw(name, b, d, h, w, ndirs, io, bc):
    """u, z, shared raw delta and `ndirs` parameter sets (the bidirectional
    recipe drawn twice, then trimmed)."""
    seed = zlib.crc32(name.encode()) % 10000
    x1 = I.make_inputs(b, d, h * w, bidir=True, io_dtype=io, bc_dtype=bc, seed=seed)
    x2 = I.make_inputs(b, d, h * w, bidir=True, io_dtype=io, bc_dtype=bc, seed=seed + 1)
    return x1, (x1.dirs + x2.dirs)[:ndirs]


def run_both(name, b, d, h, w, kinds, io="f32", bc="f32", gate=True, index=None):
    x, dirs = draw(name, b, d, h, w, len(kinds), io, bc)
    xd = x.to(DEV)
    gd = [dict(delta=xd.delta, delta_bias=p.delta_bias.to(DEV), A=p.A.to(DEV), B=p.B.to(DEV), C=p.C.to(DEV),
               D=p.D.to(DEV)) for p in dirs]
    idx = None if index is None else torch.as_tensor(index, dtype=torch.int32).to(DEV)
    got = sscan.multi(xd.u, xd.z if gate else None, gd, kinds, h, w, index=idx)
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    od = [dict(delta=x64["delta"], A=I.f64(p.A), B=I.f64(p.B), C=I.f64(p.C), D=I.f64(p.D),
               delta_bias=I.f64(p.delta_bias)) for p in dirs]
    ref = orders.scan_multi(x64["u"], x64["z"] if gate else None, od, kinds, h, w,
                            index=None if index is None else np.asarray(index), nthreads=NTHREADS)
    m = metrics(I.f64(got.cpu()), ref)
    print(f"{name}: floored {m['floored_max']:.3e}", flush=True)
    assert m["floored_max"] <= TOL[io], (name, m)


R, RR, C, CR, X, XR = (sscan.ORDER_ROW, sscan.ORDER_ROW_REV, sscan.ORDER_COL, sscan.ORDER_COL_REV,
                       sscan.ORDER_INDEX, sscan.ORDER_INDEX_REV)

CASES = [
    # name, batch, dim, height, width, kinds, io, bc, gate
    ("cross4-small", 2, 64, 8, 12, [R, RR, C, CR], "f32", "f32", True),
    ("cross4-segmented", 1, 64, 64, 64, [R, RR, C, CR], "f32", "f32", True),
    ("cross4-ragged-map", 2, 70, 5, 37, [R, RR, C, CR], "f32", "f32", True),
    ("col-only", 2, 64, 16, 9, [C], "f32", "f32", True),
    ("col-rev-only", 2, 64, 16, 9, [CR], "f32", "f32", True),
    ("row-and-col", 1, 96, 33, 31, [R, C], "f32", "f32", False),
    ("cross4-bf16", 2, 128, 32, 48, [CR, R, C, RR], "bf16", "bf16", True),
    # odd sides: the bf16 column family's element-pair kernels do not apply
    ("cross4-bf16-odd-map", 2, 64, 17, 33, [R, RR, C, CR], "bf16", "bf16", True),
    ("col-pair-bf16-no-gate", 1, 64, 32, 20, [C, CR], "bf16", "bf16", False),
]


@pytest.mark.parametrize("name,b,d,h,w,kinds,io,bc,gate", CASES, ids=[c[0] for c in CASES])
def test_multi_order_parity(name, b, d, h, w, kinds, io, bc, gate):
    run_both(name, b, d, h, w, kinds, io, bc, gate)


@pytest.mark.parametrize("h,w", [(9, 9), (16, 24), (256, 256)])
def test_spiral_orders(h, w):
    """The Samba spiral (from the library's helper) forward and reversed, next to
    the row pair (256 x 256: large enough for the flat-order gather)."""
    spiral = sscan.spiral_order(h, w).numpy()
    run_both(f"spiral-{h}x{w}", 2, 64, h, w, [X, XR, R, RR], index=spiral)


def test_random_permutation_order():
    perm = np.random.default_rng(5).permutation(20 * 20)
    run_both("perm", 1, 64, 20, 20, [X], index=perm)


@pytest.mark.parametrize("h,w", [(20, 20), (256, 256)])
def test_index_entries_outside_the_map_read_as_zero(h, w):
    """The index order with entries outside [0, h*w): such a visit step reads u, delta,
    B and C as 0 (the state still decays by exp(softplus(bias) A) there) and its
    output goes nowhere, and a token no entry names gets nothing from the index
    directions -- the documented behaviour of sscan_multi for a non-permutation.
    Expected values: the fp64 oracle on the inputs gathered that way, put back at the
    named tokens.  256 x 256 takes the flat-order gather, 20 x 20 the row groups."""
    L = h * w
    rng = np.random.default_rng(h)
    index = rng.permutation(L).astype(np.int64)
    bad = rng.choice(L, size=max(3, L // 50), replace=False)
    index[bad] = rng.choice([-1, -1000, L, L + 17], size=bad.size)
    x, dirs = draw(f"bad-index-{h}", 1, 64, h, w, 2, "f32", "f32")
    xd = x.to(DEV)
    gd = [dict(delta=xd.delta, delta_bias=p.delta_bias.to(DEV), A=p.A.to(DEV), B=p.B.to(DEV), C=p.C.to(DEV),
               D=p.D.to(DEV)) for p in dirs]
    got = sscan.multi(xd.u, xd.z, gd, [X, XR], h, w, index=torch.as_tensor(index, dtype=torch.int32).to(DEV))
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    valid = (index >= 0) & (index < L)
    safe = np.where(valid, index, 0)

    def gat(a):
        a = np.asarray(a, np.float64)
        return np.ascontiguousarray(np.where(valid, a[..., safe], 0.0))

    total = np.zeros(x64["u"].shape)
    for p, rev in zip(dirs, (False, True)):
        y = oracle.sscan_fwd(gat(x64["u"]), gat(x64["delta"]), I.f64(p.A), gat(I.f64(p.B)), gat(I.f64(p.C)),
                             I.f64(p.D), None, I.f64(p.delta_bias), reverse=rev, nthreads=NTHREADS)
        total[..., index[valid]] += y[..., valid]
    zz = x64["z"]
    ref = total * (zz / (1.0 + np.exp(-zz)))
    unnamed = np.setdiff1d(np.arange(L), index[valid])
    assert unnamed.size == bad.size
    g = I.f64(got.cpu())
    assert np.all(g[..., unnamed] == 0.0)
    m = metrics(g, ref)
    print(f"bad index {h}x{w}: floored {m['floored_max']:.3e}", flush=True)
    assert m["floored_max"] <= TOL["f32"], m


def test_yolo_stage1_map_cross4():
    """The Mamba-YOLO stage-1 map (128 x 128 tokens, 192 channels, bf16) in the
    four-direction cross order (two batch rows)."""
    run_both("yolo-cross4", 2, 192, 128, 128, [R, RR, C, CR], "bf16", "bf16", True)


def test_large_map_cross4_aggregate_runs():
    """A 512 x 512 map, 192 channels, four directions: each direction pair's 64-token
    segments are grouped in aggregate runs (sscan_scan_plan).  Whole maps of sampled
    channels against the oracle."""
    b, d, h, w = 1, 192, 512, 512
    assert sscan.scan_plan(b, d, h * w, bidir=True)["run_len"] > 1
    kinds = [R, RR, C, CR]
    x, dirs = draw("large-cross4", b, d, h, w, len(kinds), "bf16", "bf16")
    xd = x.to(DEV)
    gd = [dict(delta=xd.delta, delta_bias=p.delta_bias.to(DEV), A=p.A.to(DEV), B=p.B.to(DEV), C=p.C.to(DEV),
               D=p.D.to(DEV)) for p in dirs]
    got = sscan.multi(xd.u, xd.z, gd, kinds, h, w)
    torch.cuda.synchronize()
    rows = [0, 100, 191]
    sl = lambda t: I.f64(t[:, rows].contiguous())  # sliced before widening
    od = [dict(delta=sl(x.delta), A=I.f64(p.A[rows].contiguous()), B=I.f64(p.B), C=I.f64(p.C),
               D=I.f64(p.D[rows].contiguous()), delta_bias=I.f64(p.delta_bias[rows].contiguous())) for p in dirs]
    ref = orders.scan_multi(sl(x.u), sl(x.z), od, kinds, h, w, nthreads=NTHREADS)
    m = metrics(I.f64(got.cpu()[:, rows]), ref)
    print(f"large-cross4 rows {rows}: floored {m['floored_max']:.3e}", flush=True)
    assert m["floored_max"] <= TOL["bf16"], m
