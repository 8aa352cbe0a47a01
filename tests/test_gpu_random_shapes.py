"""GPU parity over a seeded list of random shapes and options (forward and
backward) against the fp64 oracle: batch, channels and length drawn so that the
calls land on every planning path (four lanes per channel, one segment, segments
with and without aggregate runs, ragged tiles, windows and channel groups, idle
lanes), with random dtypes, directions, reverse, gate, softplus and A recipe.
The list is fixed by its seed: the same cases run every time.
"""
import os

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


def draw_cases(seed, n, max_elems):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        b = int(rng.integers(1, 6))
        d = int(rng.choice([1, 7, 33, 64, 65, 100, 130, 192, 257]))
        L = int(rng.choice([1, 2, 15, 31, 33, 97, 200, 256, 257, 511, 777, 1500, 2900]))
        if b * d * L > max_elems:
            continue
        io = str(rng.choice(["f32", "bf16"]))
        bc = str(rng.choice(["f32", "bf16"]))
        cases.append(dict(b=b, d=d, L=L, bidir=bool(rng.integers(0, 2)), io=io, bc=bc,
                          reverse=bool(rng.integers(0, 2)), gate=bool(rng.integers(0, 4) > 0),
                          softplus=bool(rng.integers(0, 5) > 0), a_init=str(rng.choice(["s4d", "random"])),
                          seed=int(rng.integers(0, 1 << 30))))
    return cases


def draw(c):
    x = I.make_inputs(c["b"], c["d"], c["L"], bidir=c["bidir"], io_dtype=c["io"], bc_dtype=c["bc"], seed=c["seed"],
                      a_init=c["a_init"])
    if not c["softplus"]:
        # without softplus the step is delta + bias itself: keep it positive
        x.delta.abs_().add_(0.01)
        for p in x.dirs:
            p.delta_bias.zero_()
    return x


def name(c):
    return (f"b{c['b']}-d{c['d']}-L{c['L']}-{'bi' if c['bidir'] else ('rev' if c['reverse'] else 'fwd')}-"
            f"{c['io']}-{c['bc']}-{'z' if c['gate'] else 'noz'}-{'sp' if c['softplus'] else 'nosp'}-{c['a_init']}")


FWD = draw_cases(2024, 40, 1_500_000)
BWD = draw_cases(2025, 16, 400_000)


@pytest.mark.parametrize("c", FWD, ids=[name(c) for c in FWD])
def test_random_forward(c):
    x = draw(c)
    xd = x.to(DEV)
    z = xd.z if c["gate"] else None
    if c["bidir"]:
        mk = lambda p: dict(delta=xd.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D)
        y = sscan.bidir(xd.u, z, mk(xd.dirs[0]), mk(xd.dirs[1]), softplus=c["softplus"])
    else:
        p = xd.dirs[0]
        y = sscan.fwd(xd.u, xd.delta, p.A, p.B, p.C, p.D, z, p.delta_bias, softplus=c["softplus"],
                      reverse=c["reverse"])
    torch.cuda.synchronize()
    ref = oracle.run_inputs(I.as_f64_dict(x), softplus=c["softplus"], nthreads=NTHREADS,
                            reverse=c["reverse"] and not c["bidir"], gate=c["gate"])
    m = metrics(I.f64(y.cpu()), ref)
    print(name(c), f"{m['floored_max']:.3e}", flush=True)
    assert m["floored_max"] <= TOL[c["io"]], m


@pytest.mark.parametrize("c", BWD, ids=[name(c) for c in BWD])
def test_random_backward(c):
    x = draw(c)
    xd = x.to(DEV)
    rng = np.random.default_rng(c["seed"] + 1)
    g = torch.from_numpy(rng.standard_normal((c["b"], c["d"], c["L"]), dtype=np.float32)).to(x.u.dtype)
    z = xd.z if c["gate"] else None
    mk = lambda p: dict(delta=xd.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D)
    if c["bidir"]:
        r = sscan.bidir_bwd(xd.u, z, g.to(DEV), mk(xd.dirs[0]), mk(xd.dirs[1]), softplus=c["softplus"])
        got = {"du": r["du"], "dz": r["dz"], "dirs": [r["fwd"], r["rev"]]}
    else:
        p = xd.dirs[0]
        r = sscan.bwd(xd.u, xd.delta, p.A, p.B, p.C, g.to(DEV), D=p.D, z=z, delta_bias=p.delta_bias,
                      softplus=c["softplus"], reverse=c["reverse"])
        got = {"du": r["du"], "dz": r["dz"], "dirs": [r]}
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    dirs = [dict(delta=x64["delta"], **q) for q in x64["dirs"]]
    ref = oracle.sscan_bwd(x64["u"], x64["z"] if c["gate"] else None, I.f64(g), dirs, softplus=c["softplus"],
                           reverse=c["reverse"] and not c["bidir"], nthreads=NTHREADS)
    pairs = [("du", got["du"], ref["du"])]
    if c["gate"]:
        pairs.append(("dz", got["dz"], ref["dz"]))
    for k, (gd, rd) in enumerate(zip(got["dirs"], ref["dirs"])):
        pairs += [(f"dir{k}.{n}", gd[n], rd[n]) for n in ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")]
    for what, a, b in pairs:
        tol = TOL["bf16" if a.dtype == torch.bfloat16 else "f32"]
        m = metrics(I.f64(a.cpu()), b)
        assert m["floored_max"] <= tol, (name(c), what, m)
