"""GPU parity of the backward of the multi-order scan (``sscan_multi_bwd``) against
the fp64 oracle orders.scan_multi_bwd (pinned in test_oracle_orders_pins.py by
reverse-mode differentiation and central differences).

Every gradient is compared element by element with the floored relative error of
tests/parity.py at the bound of its storage dtype (1e-4 float32, 2e-2 bfloat16).
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
GRADS = ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")
R, RR, C, CR, X, XR = (sscan.ORDER_ROW, sscan.ORDER_ROW_REV, sscan.ORDER_COL, sscan.ORDER_COL_REV,
                       sscan.ORDER_INDEX, sscan.ORDER_INDEX_REV)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    sscan.load_library()  # raises if the extension is missing: no fallback
    if not os.path.exists(oracle.LIB):
        oracle.build(force=True)


def draw(name, b, d, h, w, ndirs, io, bc, shared_delta=True):
    """u, z, dout and `ndirs` parameter sets; every direction reads the same delta
    tensor unless `shared_delta` is false (then each has its own)."""
    seed = zlib.crc32(name.encode()) % 10000
    xs = [I.make_inputs(b, d, h * w, bidir=True, io_dtype=io, bc_dtype=bc, seed=seed + k) for k in range(3)]
    dirs = []
    for k in range(ndirs):
        x = xs[k // 2]
        p = x.dirs[k % 2]
        dirs.append(dict(delta=xs[0].delta if shared_delta else x.delta if k % 2 == 0 else xs[2].delta,
                         A=p.A, B=p.B, C=p.C, D=p.D, delta_bias=p.delta_bias))
    rng = np.random.default_rng(seed)
    dout = torch.from_numpy(rng.standard_normal((b, d, h * w), dtype=np.float32)).to(xs[0].u.dtype)
    return xs[0].u, xs[0].z, dout, dirs


def check(got, ref, what):
    tol = TOL["bf16" if got.dtype == torch.bfloat16 else "f32"]
    m = metrics(I.f64(got.cpu()), ref)
    print(f"{what}: floored {m['floored_max']:.3e} normwise {m['normwise']:.3e}", flush=True)
    assert m["floored_max"] <= tol, (what, m)


def run_both(name, b, d, h, w, kinds, io="f32", bc="f32", gate=True, index=None, shared_delta=True, rows=None):
    u, z, dout, dirs = draw(name, b, d, h, w, len(kinds), io, bc, shared_delta)
    dv = lambda t: None if t is None else t.to(DEV)
    gd = [{k: dv(v) for k, v in p.items()} for p in dirs]
    idx = None if index is None else torch.as_tensor(index, dtype=torch.int32).to(DEV)
    print(f"{name}: sscan_multi_bwd b={b} d={d} map={h}x{w} kinds={kinds} io={io} bc={bc}", flush=True)
    got = sscan.multi_bwd(dv(u), dv(z) if gate else None, dv(dout), gd, kinds, h, w, index=idx)
    torch.cuda.synchronize()
    # rows: compare these channels only (the oracle on a channel slice is the same
    # computation: channels do not interact)
    ch = slice(None) if rows is None else rows
    sl = lambda t: I.f64(t[:, ch].contiguous())
    od = [dict(delta=sl(p["delta"]), A=I.f64(p["A"][ch].contiguous()), B=I.f64(p["B"]), C=I.f64(p["C"]),
               D=I.f64(p["D"][ch].contiguous()), delta_bias=I.f64(p["delta_bias"][ch].contiguous())) for p in dirs]
    ref = orders.scan_multi_bwd(sl(u), sl(z) if gate else None, sl(dout), od, kinds, h, w,
                                index=None if index is None else np.asarray(index), nthreads=NTHREADS)
    pick = lambda t: t.cpu()[:, ch] if rows is not None else t.cpu()
    check(pick(got["du"]), ref["du"], f"{name} du")
    if gate:
        check(pick(got["dz"]), ref["dz"], f"{name} dz")
    else:
        assert got["dz"] is None
    for k in range(len(kinds)):
        g, r = got["dirs"][k], ref["dirs"][k]
        check(pick(g["ddelta"]), r["ddelta"], f"{name} dir{k} ddelta")
        for n in ("ddelta_bias", "dD"):
            check(g[n].cpu()[ch], r[n], f"{name} dir{k} {n}")
        check(g["dA"].cpu()[ch], r["dA"], f"{name} dir{k} dA")
        if rows is None:  # dB, dC sum over all channels
            check(g["dB"], r["dB"], f"{name} dir{k} dB")
            check(g["dC"], r["dC"], f"{name} dir{k} dC")
    return got


CASES = [
    # name, batch, dim, height, width, kinds, io, bc, gate, shared delta
    ("cross4-small", 2, 64, 8, 12, [R, RR, C, CR], "f32", "f32", True, True),
    ("cross4-own-deltas", 2, 64, 8, 12, [R, RR, C, CR], "f32", "f32", True, False),
    ("cross4-ragged-map", 2, 70, 5, 37, [R, RR, C, CR], "f32", "f32", True, False),
    ("cross4-many-windows", 1, 64, 40, 40, [CR, R, C, RR], "f32", "f32", True, True),
    ("col-only", 2, 64, 16, 9, [C], "f32", "f32", True, True),
    ("col-rev-only-no-gate", 2, 64, 16, 9, [CR], "f32", "f32", False, True),
    ("row-and-col", 1, 96, 33, 31, [R, C], "f32", "f32", False, False),
    ("rows-only", 2, 64, 10, 20, [R, RR], "f32", "f32", True, False),
    ("cross4-bf16", 2, 128, 32, 48, [CR, R, C, RR], "bf16", "bf16", True, True),
    # odd sides: the bf16 column family's element-pair kernels do not apply
    ("cross4-bf16-odd-map", 2, 64, 17, 33, [R, RR, C, CR], "bf16", "bf16", True, False),
    ("col-pair-bf16-no-gate", 1, 64, 32, 20, [C, CR], "bf16", "f32", False, True),
]


@pytest.mark.parametrize("name,b,d,h,w,kinds,io,bc,gate,shared", CASES, ids=[c[0] for c in CASES])
def test_multi_bwd_parity(name, b, d, h, w, kinds, io, bc, gate, shared):
    run_both(name, b, d, h, w, kinds, io, bc, gate, shared_delta=shared)


@pytest.mark.parametrize("h,w,io", [(9, 9, "f32"), (16, 24, "bf16")])
def test_multi_bwd_spiral_all_six(h, w, io):
    """All six orders, the index pair along the Samba spiral."""
    spiral = sscan.spiral_order(h, w).numpy()
    run_both(f"six-{h}x{w}-{io}", 2, 64, h, w, [X, XR, R, RR, C, CR], io, io, True, index=spiral,
             shared_delta=False)


def test_multi_bwd_random_permutation():
    perm = np.random.default_rng(9).permutation(20 * 20)
    run_both("perm-rev", 1, 64, 20, 20, [XR], index=perm)


def test_multi_bwd_yolo_stage1_cross4():
    """The Mamba-YOLO stage-1 map (128 x 128 tokens, 192 channels, bf16) in the
    four-direction cross order; three sampled channels against the oracle (dB and dC
    sum over all channels and are covered by the full-map cases above)."""
    run_both("yolo-cross4-bwd", 1, 192, 128, 128, [R, RR, C, CR], "bf16", "bf16", True, rows=[0, 97, 191])


def test_multi_bwd_is_bitwise_reproducible():
    u, z, dout, dirs = draw("repro", 2, 64, 24, 24, 4, "bf16", "bf16")
    dv = lambda t: t.to(DEV)
    gd = [{k: dv(v) for k, v in p.items()} for p in dirs]
    a = sscan.multi_bwd(dv(u), dv(z), dv(dout), gd, [R, RR, C, CR], 24, 24)
    b = sscan.multi_bwd(dv(u), dv(z), dv(dout), gd, [R, RR, C, CR], 24, 24)
    torch.cuda.synchronize()
    assert torch.equal(a["du"], b["du"]) and torch.equal(a["dz"], b["dz"])
    for ga, gb in zip(a["dirs"], b["dirs"]):
        for n in GRADS:
            assert torch.equal(ga[n], gb[n]), n


def test_multi_bwd_empty_map_zeroes_parameter_gradients():
    u, z, dout, dirs = draw("empty", 2, 64, 4, 4, 2, "f32", "f32")
    dv = lambda t: t.to(DEV)
    e = lambda t: t[..., :0].contiguous()
    gd = [dict(delta=e(dv(p["delta"])), A=dv(p["A"]), B=e(dv(p["B"])), C=e(dv(p["C"])), D=dv(p["D"]),
               delta_bias=dv(p["delta_bias"])) for p in dirs]
    got = sscan.multi_bwd(e(dv(u)), e(dv(z)), e(dv(dout)), gd, [C, CR], 0, 4)
    torch.cuda.synchronize()
    for g in got["dirs"]:
        for n in ("dA", "dD", "ddelta_bias"):
            assert torch.count_nonzero(g[n]).item() == 0, n
