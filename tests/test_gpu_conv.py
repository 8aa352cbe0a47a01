"""GPU parity of the front-end convolution: ``sscan_conv1d`` and the scan with the
convolution fused in (``sscan_fwd_conv``, ``sscan_bidir_conv``) against the fp64
oracle (conv pinned in test_oracle_conv_pins.py, the scan in test_oracle_pins.py).
"""
import os
import zlib

import numpy as np
import pytest
import torch

from oracle import oracle
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


def check(got, ref, tol, what):
    m = metrics(I.f64(got.cpu()), ref)
    print(f"{what}: floored {m['floored_max']:.3e}", flush=True)
    assert m["floored_max"] <= tol, (what, m)


def conv_params(name, d, width, same, silu, bias=True):
    rng = np.random.default_rng(zlib.crc32(name.encode()) % 1000)
    w = torch.from_numpy(rng.normal(0.0, 0.5, (d, width))).float()
    b = torch.from_numpy(rng.normal(0.0, 0.2, d)).float() if bias else None
    return dict(weight=w, bias=b, same=same, silu=silu)


CONV_CASES = [
    # name, batch, dim, len, width, same, silu, io
    ("w4-causal", 2, 64, 100, 4, False, False, "f32"),
    ("w3-causal-silu", 2, 70, 37, 3, False, True, "f32"),
    ("w2-causal", 1, 5, 9, 2, False, False, "f32"),
    ("w1", 2, 8, 16, 1, False, False, "f32"),
    ("w3-same", 3, 64, 197, 3, True, False, "f32"),
    ("w1-same-silu", 1, 64, 20, 1, True, True, "f32"),
    ("w4-bf16", 2, 128, 1000, 4, False, True, "bf16"),
    ("w3-same-bf16", 2, 64, 197, 3, True, False, "bf16"),
    ("short-len2", 2, 64, 2, 4, False, False, "f32"),
]


@pytest.mark.parametrize("name,b,d,L,width,same,silu,io", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_conv1d_parity(name, b, d, L, width, same, silu, io):
    x = I.make_inputs(b, d, L, io_dtype=io, seed=zlib.crc32(name.encode()) % 10000)
    cp = conv_params(name, d, width, same, silu, bias=(width != 2))
    got = sscan.conv1d(x.u.to(DEV), cp["weight"].to(DEV), None if cp["bias"] is None else cp["bias"].to(DEV),
                       same=same, silu=silu)
    torch.cuda.synchronize()
    ref = oracle.conv1d(I.f64(x.u), I.f64(cp["weight"]), None if cp["bias"] is None else I.f64(cp["bias"]),
                        same=same, silu=silu)
    check(got, ref, TOL[io], f"conv1d {name}")


FUSED_CASES = [
    # name, batch, dim, len, bidir, io, bc, width, same, silu, reverse
    ("short", 2, 64, 100, False, "f32", "f32", 4, False, False, False),
    ("short-rev-silu", 2, 70, 77, False, "f32", "f32", 4, False, True, True),
    ("segmented", 2, 96, 3000, False, "f32", "f32", 4, False, True, False),
    ("segmented-rev", 1, 64, 2500, False, "f32", "f32", 3, False, False, True),
    ("bf16-long", 1, 128, 5000, False, "bf16", "f32", 4, False, True, False),
    ("bidir-same3", 2, 64, 197, True, "f32", "f32", 3, True, False, False),
    ("bidir-segmented", 1, 64, 1003, True, "bf16", "bf16", 4, False, True, False),
]


def oracle_fused(x, cp, reverse=False):
    x64 = I.as_f64_dict(x)
    u = oracle.conv1d(x64["u"], I.f64(cp["weight"]), I.f64(cp["bias"]), cp["same"], cp["silu"])
    x64 = dict(x64, u=u)
    return oracle.run_inputs(x64, nthreads=NTHREADS, reverse=reverse)


def gpu_fused(xd, cp, reverse=False):
    c = dict(weight=cp["weight"].to(DEV), bias=cp["bias"].to(DEV), same=cp["same"], silu=cp["silu"])
    if len(xd.dirs) == 1:
        p = xd.dirs[0]
        return sscan.fwd_conv(xd.u, c, xd.delta, p.A, p.B, p.C, p.D, xd.z, p.delta_bias, reverse=reverse)
    mk = lambda p: dict(delta=xd.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D)
    return sscan.bidir_conv(xd.u, c, xd.z, mk(xd.dirs[0]), mk(xd.dirs[1]))


@pytest.mark.parametrize("name,b,d,L,bidir,io,bc,width,same,silu,reverse", FUSED_CASES,
                         ids=[c[0] for c in FUSED_CASES])
def test_fused_scan_parity(name, b, d, L, bidir, io, bc, width, same, silu, reverse):
    x = I.make_inputs(b, d, L, bidir=bidir, io_dtype=io, bc_dtype=bc, seed=zlib.crc32(name.encode()) % 10000)
    cp = conv_params(name, d, width, same, silu)
    got = gpu_fused(x.to(DEV), cp, reverse)
    torch.cuda.synchronize()
    check(got, oracle_fused(x, cp, reverse), TOL[io], f"fused {name}")


@pytest.mark.parametrize("bidir", [False, True])
def test_fused_equals_conv_then_scan_f32(bidir):
    """In float32 the fused front-end computes exactly the values sscan_conv1d
    stores, so the fused call and conv1d followed by the plain scan agree bitwise."""
    b, d, L = 2, 96, 1500
    x = I.make_inputs(b, d, L, bidir=bidir, seed=31 + bidir)
    cp = conv_params("bitwise", d, 4, False, True)
    xd = x.to(DEV)
    fused = gpu_fused(xd, cp)
    u = sscan.conv1d(xd.u, cp["weight"].to(DEV), cp["bias"].to(DEV), silu=True)
    xu = I.ScanInputs(u, xd.delta, xd.z, xd.dirs, xd.io_dtype, xd.bc_dtype)
    plain = sscan.run_inputs(xu)
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)


# --- backward through the convolution (sscan_bwd_conv, sscan_bidir_bwd_conv) ----------------------

BWD_CONV_CASES = [
    # name, batch, dim, len, bidir, io, bc, width, same, silu, reverse
    ("bwd-w4-silu", 2, 64, 100, False, "f32", "f32", 4, False, True, False),
    ("bwd-w3-rev", 2, 70, 77, False, "f32", "f32", 3, False, False, True),
    ("bwd-segmented-bf16", 1, 128, 3000, False, "bf16", "f32", 4, False, True, False),
    ("bwd-bidir-same3", 2, 64, 197, True, "f32", "f32", 3, True, False, False),
    ("bwd-bidir-bf16", 1, 96, 1003, True, "bf16", "bf16", 4, False, True, False),
    ("bwd-w1-same", 2, 40, 50, False, "f32", "f32", 1, True, True, False),
]


@pytest.mark.parametrize("name,b,d,L,bidir,io,bc,width,same,silu,reverse", BWD_CONV_CASES,
                         ids=[c[0] for c in BWD_CONV_CASES])
def test_bwd_conv_parity(name, b, d, L, bidir, io, bc, width, same, silu, reverse):
    """Every gradient of the backward through the convolution against the oracle
    (the scan's backward at u = conv(x), then the convolution's backward).  The
    kernels recompute u in fp32 as the fused forward computes it; a bf16 call is
    held to the bf16 bound in all its gradients (its inputs and stored gradients
    are bf16), float32 calls to 1e-4."""
    seed = zlib.crc32(name.encode()) % 10000
    x = I.make_inputs(b, d, L, bidir=bidir, io_dtype=io, bc_dtype=bc, seed=seed)
    cp = conv_params(name, d, width, same, silu)
    rng = np.random.default_rng(seed + 1)
    dout = torch.from_numpy(rng.standard_normal((b, d, L), dtype=np.float32)).to(x.u.dtype)
    xd = x.to(DEV)
    c = dict(weight=cp["weight"].to(DEV), bias=cp["bias"].to(DEV), same=same, silu=silu)
    mk = lambda p: dict(delta=xd.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D)
    if bidir:
        r = sscan.bidir_bwd_conv(xd.u, c, xd.z, dout.to(DEV), mk(xd.dirs[0]), mk(xd.dirs[1]))
        got_dirs = [r["fwd"], r["rev"]]
    else:
        p = xd.dirs[0]
        r = sscan.bwd_conv(xd.u, c, xd.delta, p.A, p.B, p.C, dout.to(DEV), D=p.D, z=xd.z, delta_bias=p.delta_bias,
                           reverse=reverse)
        got_dirs = [r]
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    dirs = [dict(delta=x64["delta"], A=q["A"], B=q["B"], C=q["C"], D=q["D"], delta_bias=q["delta_bias"])
            for q in x64["dirs"]]
    ref = oracle.sscan_bwd_conv(x64["u"], I.f64(cp["weight"]), I.f64(cp["bias"]), same, silu, x64["z"], I.f64(dout),
                                dirs, reverse=reverse, nthreads=NTHREADS)
    tol = TOL[io]
    for k in ("dx", "dz", "dconv_w", "dconv_b"):
        check(r[k], ref[k], tol, f"{name} {k}")
    for k, (gd, rd) in enumerate(zip(got_dirs, ref["dirs"])):
        for gname in ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD"):
            check(gd[gname], rd[gname], tol, f"{name} dir{k} {gname}")


def test_bwd_conv_deterministic():
    x = I.make_inputs(2, 96, 700, io_dtype="bf16", bc_dtype="bf16", seed=71)
    cp = conv_params("det", 96, 4, False, True)
    xd = x.to(DEV)
    c = dict(weight=cp["weight"].to(DEV), bias=cp["bias"].to(DEV), silu=True)
    dout = torch.randn(x.u.shape, generator=torch.Generator().manual_seed(5)).to(x.u.dtype).to(DEV)
    p = xd.dirs[0]
    run = lambda: sscan.bwd_conv(xd.u, c, xd.delta, p.A, p.B, p.C, dout, D=p.D, z=xd.z, delta_bias=p.delta_bias)
    a, b = run(), run()
    torch.cuda.synchronize()
    for k in ("dx", "dz", "dconv_w", "dconv_b", "dA", "dB"):
        assert torch.equal(a[k], b[k]), k
