"""GPU parity of the backward pass (``sscan_bwd``, ``sscan_bidir_bwd``) against the
fp64 backward oracle (pinned in test_oracle_bwd_pins.py).

Every gradient is compared element by element with the floored relative error of
tests/parity.py, at the bound of its storage dtype (1e-4 float32, 2e-2 bfloat16):
du, dz, ddelta in the I/O dtype, dB and dC in B/C's dtype, dA, dD and delta_bias in
float32.
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
GRADS = ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    sscan.load_library()  # raises if the extension is missing: no fallback
    if not os.path.exists(oracle.LIB):
        oracle.build(force=True)


def _dtype_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def check(got, ref, what):
    assert got is not None and ref is not None, what
    tol = TOL[_dtype_name(got)]
    m = metrics(I.f64(got.cpu()), ref)
    print(f"{what}: floored {m['floored_max']:.3e} normwise {m['normwise']:.3e}", flush=True)
    assert m["floored_max"] <= tol, (what, m)


def make_dout(x, seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(tuple(x.u.shape), dtype=np.float32)
    return torch.from_numpy(g).to(x.u.dtype)


def oracle_grads(x, dout, softplus=True, gate=True, reverse=False, opt=True):
    x64 = I.as_f64_dict(x)
    dirs = []
    for p in x64["dirs"]:
        q = dict(delta=x64["delta"], A=p["A"], B=p["B"], C=p["C"])
        if opt:
            q.update(D=p["D"], delta_bias=p["delta_bias"])
        dirs.append(q)
    return oracle.sscan_bwd(x64["u"], x64["z"] if gate else None, I.f64(dout), dirs, softplus=softplus,
                            reverse=reverse, nthreads=NTHREADS)


def gpu_grads(x, dout, softplus=True, gate=True, reverse=False, opt=True):
    xd = x.to(DEV)
    z = xd.z if gate else None
    g = dout.to(DEV)
    mk = lambda p: dict(delta=xd.delta, A=p.A, B=p.B, C=p.C, D=p.D if opt else None,
                        delta_bias=p.delta_bias if opt else None)
    if len(xd.dirs) == 1:
        p = mk(xd.dirs[0])
        r = sscan.bwd(xd.u, p["delta"], p["A"], p["B"], p["C"], g, D=p["D"], z=z, delta_bias=p["delta_bias"],
                      softplus=softplus, reverse=reverse)
        out = {"du": r["du"], "dz": r["dz"], "dirs": [{k: r[k] for k in GRADS}]}
    else:
        r = sscan.bidir_bwd(xd.u, z, g, mk(xd.dirs[0]), mk(xd.dirs[1]), softplus=softplus)
        out = {"du": r["du"], "dz": r["dz"], "dirs": [r["fwd"], r["rev"]]}
    torch.cuda.synchronize()
    return out


def compare(got, ref, name, gate=True, opt=True):
    check(got["du"], ref["du"], f"{name} du")
    if gate:
        check(got["dz"], ref["dz"], f"{name} dz")
    for k, (gd, rd) in enumerate(zip(got["dirs"], ref["dirs"])):
        for g in GRADS:
            if not opt and g in ("ddelta_bias", "dD"):
                assert gd[g] is None and rd[g] is None
                continue
            check(gd[g], rd[g], f"{name} dir{k} {g}")


CASES = [
    # name, batch, dim, len, bidir, io, bc, kwargs
    ("one-window", 2, 64, 32, False, "f32", "f32", {}),
    ("ragged-windows", 2, 70, 100, False, "f32", "f32", {}),
    ("ragged-windows-rev", 2, 70, 100, False, "f32", "f32", dict(reverse=True)),
    ("len1", 3, 64, 1, False, "f32", "f32", {}),
    ("many-windows", 2, 96, 1000, False, "f32", "f32", {}),
    ("many-windows-rev", 1, 130, 777, False, "f32", "f32", dict(reverse=True)),
    ("bf16", 2, 64, 300, False, "bf16", "bf16", {}),
    ("bf16-f32bc", 1, 128, 2000, False, "bf16", "f32", {}),
    ("no-gate", 2, 64, 100, False, "f32", "f32", dict(gate=False)),
    ("no-softplus", 2, 64, 100, False, "f32", "f32", dict(softplus=False)),
    ("no-D-bias", 2, 64, 100, False, "f32", "f32", dict(opt=False)),
    ("bidir", 2, 64, 197, True, "f32", "f32", {}),
    ("bidir-ragged-dim", 3, 70, 61, True, "f32", "f32", {}),
    ("bidir-bf16", 2, 128, 500, True, "bf16", "bf16", {}),
    ("bidir-no-gate", 2, 64, 40, True, "f32", "f32", dict(gate=False)),
    # 51 channel groups (the last one partial) over three window-pass blocks
    ("bidir-split-ragged", 2, 202, 150, True, "bf16", "bf16", {}),
]


@pytest.mark.parametrize("name,b,d,L,bidir,io,bc,kw", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(name, b, d, L, bidir, io, bc, kw):
    seed = zlib.crc32(name.encode()) % 10000
    x = I.make_inputs(b, d, L, bidir=bidir, io_dtype=io, bc_dtype=bc, seed=seed)
    if not kw.get("softplus", True):
        x.delta.abs_().add_(0.01)
        for p in x.dirs:
            p.delta_bias.zero_()
    dout = make_dout(x, seed + 1)
    compare(gpu_grads(x, dout, **kw), oracle_grads(x, dout, **kw), name, kw.get("gate", True), kw.get("opt", True))


@pytest.mark.parametrize("a_init", ["s4d", "random"])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_bwd_config_full(cfg, a_init):
    x = I.config_inputs(cfg, 0, a_init=a_init)
    dout = make_dout(x, 77 + cfg)
    compare(gpu_grads(x, dout), oracle_grads(x, dout), f"config {cfg} A {a_init}")


@pytest.mark.parametrize("a_init", ["s4d", "random"])
def test_bwd_long_sequence(a_init):
    """The long-sequence workload's shape and launch configuration (8192 windows
    of one row): per-channel gradients on sampled channels of the full call, and
    dB/dC (sums over all channels) on a 64-channel slice at the full length."""
    x = I.config_inputs(4, 0, a_init=a_init)
    dout = make_dout(x, 81)
    got = gpu_grads(x, dout)
    x64 = I.as_f64_dict(x)
    p = x64["dirs"][0]
    rows = [0, 63, 64, 777, 1535]
    for d in rows:
        sl = lambda a: a[:, d:d + 1]
        ref = oracle.sscan_bwd(sl(x64["u"]), sl(x64["z"]), I.f64(dout[:, d:d + 1]),
                               [dict(delta=sl(x64["delta"]), A=p["A"][d:d + 1], B=p["B"], C=p["C"],
                                     D=p["D"][d:d + 1], delta_bias=p["delta_bias"][d:d + 1])], nthreads=1)
        check(got["du"][:, d:d + 1], ref["du"], f"row {d} du")
        check(got["dz"][:, d:d + 1], ref["dz"], f"row {d} dz")
        g0, r0 = got["dirs"][0], ref["dirs"][0]
        check(g0["ddelta"][:, d:d + 1], r0["ddelta"], f"row {d} ddelta")
        cond = np.abs(r0["ddelta"]).sum() / abs(r0["ddelta"].sum())
        print(f"row {d} delta_bias condition number {cond:.3g}", flush=True)
        for k in ("dA", "dD", "ddelta_bias"):
            check(g0[k][d:d + 1], r0[k], f"row {d} {k}")
    # a 64-channel slice at full length: every gradient, dB and dC included
    xs = I.ScanInputs(x.u[:, :64].contiguous(), x.delta[:, :64].contiguous(), x.z[:, :64].contiguous(),
                      [I.DirParams(q.delta_bias[:64].contiguous(), q.A[:64].contiguous(), q.B, q.C,
                                   q.D[:64].contiguous()) for q in x.dirs], x.io_dtype, x.bc_dtype)
    ds = dout[:, :64].contiguous()
    compare(gpu_grads(xs, ds), oracle_grads(xs, ds), "long 64-channel slice")


def test_bwd_deterministic():
    x = I.make_inputs(2, 96, 1000, bidir=True, io_dtype="f32", bc_dtype="f32", seed=5)
    dout = make_dout(x, 6)
    a, b = gpu_grads(x, dout), gpu_grads(x, dout)
    assert torch.equal(a["du"], b["du"]) and torch.equal(a["dz"], b["dz"])
    for ga, gb in zip(a["dirs"], b["dirs"]):
        for k in GRADS:
            assert torch.equal(ga[k], gb[k]), k


def test_bwd_empty_sequence_zeroes_parameter_grads():
    x = I.make_inputs(2, 70, 0, seed=8)
    xd = x.to(DEV)
    p = xd.dirs[0]
    g = torch.empty_like(xd.u)
    r = sscan.bwd(xd.u, xd.delta, p.A, p.B, p.C, g, D=p.D, z=xd.z, delta_bias=p.delta_bias)
    torch.cuda.synchronize()
    for k in ("dA", "dD", "ddelta_bias"):
        assert torch.count_nonzero(r[k]).item() == 0, k
    assert r["du"].numel() == 0 and r["dB"].numel() == 0


# --- state I/O: sscan_bwd_state (entry state h0, gradient of the final state, dh0) ------------

STATE_CASES = [
    # name, batch, dim, len, io, bc, reverse
    ("state-one-window", 2, 64, 30, "f32", "f32", False),
    ("state-many-windows", 2, 96, 1000, "f32", "f32", False),
    ("state-many-windows-rev", 1, 130, 777, "f32", "f32", True),
    ("state-bf16", 2, 64, 2000, "bf16", "f32", False),
    ("state-long-runs", 1, 64, 40000, "f32", "f32", True),
]


def _state_draw(name, b, d, L, io, bc):
    seed = zlib.crc32(name.encode()) % 10000
    x = I.make_inputs(b, d, L, io_dtype=io, bc_dtype=bc, seed=seed)
    rng = np.random.default_rng(seed + 5)
    h0 = torch.from_numpy(rng.normal(0.0, 1.0, (b, d, 16))).float()
    dhl = torch.from_numpy(rng.normal(0.0, 1.0, (b, d, 16))).float()
    return x, make_dout(x, seed + 1), h0, dhl


@pytest.mark.parametrize("name,b,d,L,io,bc,reverse", STATE_CASES, ids=[c[0] for c in STATE_CASES])
def test_bwd_state_parity(name, b, d, L, io, bc, reverse):
    x, dout, h0, dhl = _state_draw(name, b, d, L, io, bc)
    xd = x.to(DEV)
    p = xd.dirs[0]
    r = sscan.bwd_state(xd.u, xd.delta, p.A, p.B, p.C, dout.to(DEV), D=p.D, z=xd.z, delta_bias=p.delta_bias,
                        h0=h0.to(DEV), dh_last=dhl.to(DEV), reverse=reverse)
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    q = x64["dirs"][0]
    ref = oracle.sscan_bwd(x64["u"], x64["z"], I.f64(dout), [dict(delta=x64["delta"], A=q["A"], B=q["B"], C=q["C"],
                                                                  D=q["D"], delta_bias=q["delta_bias"])],
                           reverse=reverse, nthreads=NTHREADS, h0=h0.double().numpy(), dh_last=dhl.double().numpy(),
                           return_dh0=True)
    check(r["dh0"], ref["dh0"], f"{name} dh0")
    compare({"du": r["du"], "dz": r["dz"], "dirs": [{k: r[k] for k in GRADS}]}, ref, name)


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_state_pieces_equal_the_whole(reverse):
    """A sequence trained in two pieces: forward piece by piece with the state handed
    on, backward piece by piece in reverse order with dh0 handed back as dh_last;
    the joined gradients match the oracle's gradients of the whole sequence."""
    b, d, L, m = 2, 96, 1500, 700
    x, dout, _, _ = _state_draw(f"pieces-{reverse}", b, d, L, "f32", "f32")
    xd = x.to(DEV)
    p = xd.dirs[0]
    g = dout.to(DEV)
    first, second = (slice(m, L), slice(0, m)) if reverse else (slice(0, m), slice(m, L))
    cut = lambda t, s: t[..., s].contiguous()
    _, hmid = sscan.fwd_state(cut(xd.u, first), cut(xd.delta, first), p.A, cut(p.B, first), cut(p.C, first), p.D,
                              cut(xd.z, first), p.delta_bias, reverse=reverse)
    g2 = sscan.bwd_state(cut(xd.u, second), cut(xd.delta, second), p.A, cut(p.B, second), cut(p.C, second),
                         cut(g, second), D=p.D, z=cut(xd.z, second), delta_bias=p.delta_bias, h0=hmid, reverse=reverse)
    g1 = sscan.bwd_state(cut(xd.u, first), cut(xd.delta, first), p.A, cut(p.B, first), cut(p.C, first), cut(g, first),
                         D=p.D, z=cut(xd.z, first), delta_bias=p.delta_bias, dh_last=g2["dh0"], reverse=reverse)
    torch.cuda.synchronize()
    join = lambda a1, a2: torch.cat([a1, a2] if not reverse else [a2, a1], dim=-1)
    got = {"du": join(g1["du"], g2["du"]), "dz": join(g1["dz"], g2["dz"]),
           "dirs": [{"ddelta": join(g1["ddelta"], g2["ddelta"]), "dB": join(g1["dB"], g2["dB"]),
                     "dC": join(g1["dC"], g2["dC"]), "dA": g1["dA"] + g2["dA"], "dD": g1["dD"] + g2["dD"],
                     "ddelta_bias": g1["ddelta_bias"] + g2["ddelta_bias"]}]}
    compare(got, oracle_grads(x, dout, reverse=reverse), f"pieces reverse={reverse}")


def test_bwd_state_empty_sequence_passes_dh_last():
    b, d = 2, 70
    x, _, h0, dhl = _state_draw("state-empty", b, d, 0, "f32", "f32")
    xd = x.to(DEV)
    p = xd.dirs[0]
    r = sscan.bwd_state(xd.u, xd.delta, p.A, p.B, p.C, torch.empty_like(xd.u), D=p.D, z=xd.z,
                        delta_bias=p.delta_bias, h0=h0.to(DEV), dh_last=dhl.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(r["dh0"].cpu(), dhl)
