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


# ---- scans along several orders of a 2-D map, forward and backward --------------

def draw_maps(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        h, w = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        kinds = sorted(int(k) for k in rng.choice(6, size=int(rng.integers(1, 7)), replace=False))
        io = str(rng.choice(["f32", "bf16"]))
        out.append(dict(b=int(rng.integers(1, 4)), d=int(rng.choice([16, 64, 70, 130])), h=h, w=w, kinds=kinds,
                        io=io, bc=str(rng.choice(["f32", "bf16"])), gate=bool(rng.integers(0, 4) > 0),
                        seed=int(rng.integers(0, 1 << 30))))
    return out


MAPS = draw_maps(2026, 12)


def map_name(c):
    return f"b{c['b']}-d{c['d']}-{c['h']}x{c['w']}-k{''.join(map(str, c['kinds']))}-{c['io']}-{c['bc']}-{'z' if c['gate'] else 'noz'}"


@pytest.mark.parametrize("c", MAPS, ids=[map_name(c) for c in MAPS])
def test_random_multi_forward_and_backward(c):
    from oracle import orders

    L = c["h"] * c["w"]
    rng = np.random.default_rng(c["seed"])
    xs = [I.make_inputs(c["b"], c["d"], L, bidir=True, io_dtype=c["io"], bc_dtype=c["bc"], seed=c["seed"] + k)
          for k in range(3)]
    dirs = [dict(delta=xs[k // 2].delta, A=xs[k // 2].dirs[k % 2].A, B=xs[k // 2].dirs[k % 2].B,
                 C=xs[k // 2].dirs[k % 2].C, D=xs[k // 2].dirs[k % 2].D, delta_bias=xs[k // 2].dirs[k % 2].delta_bias)
            for k in range(len(c["kinds"]))]
    perm = rng.permutation(L)
    u, z = xs[0].u, xs[0].z
    g = torch.from_numpy(rng.standard_normal((c["b"], c["d"], L), dtype=np.float32)).to(u.dtype)
    dv = lambda t: t.to(DEV)
    gd = [{k: dv(v) for k, v in p.items()} for p in dirs]
    idx = torch.as_tensor(perm, dtype=torch.int32).to(DEV)
    zz = dv(z) if c["gate"] else None
    y = sscan.multi(dv(u), zz, gd, c["kinds"], c["h"], c["w"], index=idx)
    gr = sscan.multi_bwd(dv(u), zz, dv(g), gd, c["kinds"], c["h"], c["w"], index=idx)
    torch.cuda.synchronize()
    od = [{k: I.f64(v) for k, v in p.items()} for p in dirs]
    z64 = I.f64(z) if c["gate"] else None
    ref_y = orders.scan_multi(I.f64(u), z64, od, c["kinds"], c["h"], c["w"], index=perm, nthreads=NTHREADS)
    ref_g = orders.scan_multi_bwd(I.f64(u), z64, I.f64(g), od, c["kinds"], c["h"], c["w"], index=perm,
                                  nthreads=NTHREADS)
    pairs = [("y", y, ref_y), ("du", gr["du"], ref_g["du"])]
    if c["gate"]:
        pairs.append(("dz", gr["dz"], ref_g["dz"]))
    for k, (a, b) in enumerate(zip(gr["dirs"], ref_g["dirs"])):
        pairs += [(f"dir{k}.{n}", a[n], b[n]) for n in ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")]
    for what, a, b in pairs:
        tol = TOL["bf16" if a.dtype == torch.bfloat16 else "f32"]
        m = metrics(I.f64(a.cpu()), b)
        assert m["floored_max"] <= tol, (map_name(c), what, m)


# ---- the scan through the front-end convolution, forward and backward ------------

def draw_convs(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        same = bool(rng.integers(0, 2))
        width = int(rng.choice([1, 3])) if same else int(rng.integers(1, 5))
        out.append(dict(b=int(rng.integers(1, 4)), d=int(rng.choice([5, 64, 100])),
                        L=int(rng.choice([1, 9, 64, 200, 999])), bidir=bool(rng.integers(0, 2)),
                        reverse=bool(rng.integers(0, 2)), io=str(rng.choice(["f32", "bf16"])),
                        bc=str(rng.choice(["f32", "bf16"])), width=width, same=same, silu=bool(rng.integers(0, 2)),
                        seed=int(rng.integers(0, 1 << 30))))
    return out


CONVS = draw_convs(2027, 10)


def conv_name(c):
    return (f"b{c['b']}-d{c['d']}-L{c['L']}-{'bi' if c['bidir'] else ('rev' if c['reverse'] else 'fwd')}-{c['io']}-"
            f"{c['bc']}-w{c['width']}{'s' if c['same'] else 'c'}{'-silu' if c['silu'] else ''}")


@pytest.mark.parametrize("c", CONVS, ids=[conv_name(c) for c in CONVS])
def test_random_conv_forward_and_backward(c):
    rng = np.random.default_rng(c["seed"])
    x = I.make_inputs(c["b"], c["d"], c["L"], bidir=c["bidir"], io_dtype=c["io"], bc_dtype=c["bc"], seed=c["seed"])
    wt = torch.from_numpy(rng.normal(0.0, 0.5, (c["d"], c["width"]))).float()
    bias = torch.from_numpy(rng.normal(0.0, 0.1, c["d"])).float()
    g = torch.from_numpy(rng.standard_normal((c["b"], c["d"], c["L"]), dtype=np.float32)).to(x.u.dtype)
    xd = x.to(DEV)
    cp = dict(weight=wt.to(DEV), bias=bias.to(DEV), same=c["same"], silu=c["silu"])
    mk = lambda p: dict(delta=xd.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D)
    rev = c["reverse"] and not c["bidir"]
    if c["bidir"]:
        y = sscan.bidir_conv(xd.u, cp, xd.z, mk(xd.dirs[0]), mk(xd.dirs[1]))
        r = sscan.bidir_bwd_conv(xd.u, cp, xd.z, g.to(DEV), mk(xd.dirs[0]), mk(xd.dirs[1]))
        gdirs = [r["fwd"], r["rev"]]
    else:
        p = xd.dirs[0]
        y = sscan.fwd_conv(xd.u, cp, xd.delta, p.A, p.B, p.C, p.D, xd.z, p.delta_bias, reverse=rev)
        r = sscan.bwd_conv(xd.u, cp, xd.delta, p.A, p.B, p.C, g.to(DEV), D=p.D, z=xd.z, delta_bias=p.delta_bias,
                           reverse=rev)
        gdirs = [r]
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    dirs = [dict(delta=x64["delta"], **q) for q in x64["dirs"]]
    w64, b64 = wt.double().numpy(), bias.double().numpy()
    u64 = oracle.conv1d(x64["u"], w64, b64, same=c["same"], silu=c["silu"])
    if c["bidir"]:
        ref_y = oracle.sscan_bidir(u64, x64["z"], dirs[0], dirs[1])
    else:
        q = dirs[0]
        ref_y = oracle.sscan_fwd(u64, q["delta"], q["A"], q["B"], q["C"], q["D"], x64["z"], q["delta_bias"],
                                 reverse=rev)
    ref = oracle.sscan_bwd_conv(x64["u"], w64, b64, c["same"], c["silu"], x64["z"], I.f64(g), dirs, reverse=rev)
    pairs = [("y", y, ref_y), ("dx", r["dx"], ref["dx"]), ("dz", r["dz"], ref["dz"]),
             ("dconv_w", r["dconv_w"], ref["dconv_w"]), ("dconv_b", r["dconv_b"], ref["dconv_b"])]
    for k, (a, b) in enumerate(zip(gdirs, ref["dirs"])):
        pairs += [(f"dir{k}.{n}", a[n], b[n]) for n in ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")]
    for what, a, b in pairs:
        tol = TOL["bf16" if (a.dtype == torch.bfloat16 or c["io"] == "bf16") else "f32"]
        m = metrics(I.f64(a.cpu()), b)
        assert m["floored_max"] <= tol, (conv_name(c), what, m)


# ---- state I/O: forward with an entry state and the final state, and its backward

def draw_states(seed, n):
    rng = np.random.default_rng(seed)
    return [dict(b=int(rng.integers(1, 4)), d=int(rng.choice([3, 64, 65, 130])),
                 L=int(rng.choice([0, 1, 17, 200, 600, 1500])), reverse=bool(rng.integers(0, 2)),
                 io=str(rng.choice(["f32", "bf16"])), bc=str(rng.choice(["f32", "bf16"])),
                 h0=bool(rng.integers(0, 4) > 0), dh_last=bool(rng.integers(0, 4) > 0),
                 seed=int(rng.integers(0, 1 << 30))) for _ in range(n)]


STATES = draw_states(2028, 10)


def state_name(c):
    return (f"b{c['b']}-d{c['d']}-L{c['L']}-{'rev' if c['reverse'] else 'fwd'}-{c['io']}-{c['bc']}"
            f"{'-h0' if c['h0'] else ''}{'-dhl' if c['dh_last'] else ''}")


@pytest.mark.parametrize("c", STATES, ids=[state_name(c) for c in STATES])
def test_random_state_io_forward_and_backward(c):
    rng = np.random.default_rng(c["seed"])
    x = I.make_inputs(c["b"], c["d"], c["L"], io_dtype=c["io"], bc_dtype=c["bc"], seed=c["seed"])
    h0 = torch.from_numpy(rng.standard_normal((c["b"], c["d"], 16), dtype=np.float32)) if c["h0"] else None
    dhl = torch.from_numpy(rng.standard_normal((c["b"], c["d"], 16), dtype=np.float32)) if c["dh_last"] else None
    g = torch.from_numpy(rng.standard_normal((c["b"], c["d"], c["L"]), dtype=np.float32)).to(x.u.dtype)
    xd = x.to(DEV)
    p = xd.dirs[0]
    dv = lambda t: None if t is None else t.to(DEV)
    y, hl = sscan.fwd_state(xd.u, xd.delta, p.A, p.B, p.C, p.D, xd.z, p.delta_bias, h0=dv(h0),
                            reverse=c["reverse"])
    r = sscan.bwd_state(xd.u, xd.delta, p.A, p.B, p.C, g.to(DEV), D=p.D, z=xd.z, delta_bias=p.delta_bias,
                        h0=dv(h0), dh_last=dv(dhl), reverse=c["reverse"])
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    q = x64["dirs"][0]
    h064 = I.f64(h0) if c["h0"] else None
    ref_y, ref_h = oracle.sscan_fwd(x64["u"], x64["delta"], q["A"], q["B"], q["C"], q["D"], x64["z"],
                                    q["delta_bias"], reverse=c["reverse"], h0=h064, return_last_state=True,
                                    nthreads=NTHREADS)
    ref = oracle.sscan_bwd(x64["u"], x64["z"], I.f64(g), [dict(delta=x64["delta"], **q)], reverse=c["reverse"],
                           h0=h064, dh_last=I.f64(dhl) if c["dh_last"] else None, return_dh0=True,
                           nthreads=NTHREADS)
    pairs = [("y", y, ref_y), ("h_last", hl, ref_h), ("du", r["du"], ref["du"]), ("dz", r["dz"], ref["dz"]),
             ("dh0", r["dh0"], ref["dh0"])]
    pairs += [(n, r[n], ref["dirs"][0][n]) for n in ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")]
    for what, a, b in pairs:
        if b is None or np.asarray(b).size == 0:
            continue
        # the bound of the stored dtype (the oracle reads the same bf16 input values)
        tol = TOL["bf16" if a.dtype == torch.bfloat16 else "f32"]
        m = metrics(I.f64(a.cpu()), b)
        assert m["floored_max"] <= tol, (state_name(c), what, m)
