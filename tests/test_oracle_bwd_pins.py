"""Pins of the fp64 backward oracle (oracle/sscan_oracle_bwd.c).

The gradients are checked against two things the derivation in that file does not
share: central finite differences of the forward oracle (itself pinned in
test_oracle_pins.py), and PyTorch's reverse-mode differentiation (a library
routine) through a plain fp64 token-by-token recurrence.  No HIP code is involved.
"""
import numpy as np
import pytest
import torch

from oracle import oracle

NAMES = ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")


def _case(rng, b, d, L, N=16, dt_scale=1.0):
    p = dict(
        delta=rng.normal(0.0, 0.5, (b, d, L)),
        A=-np.exp(rng.uniform(-1.0, 1.5, (d, N))),
        B=rng.normal(size=(b, N, L)),
        C=rng.normal(size=(b, N, L)),
        D=rng.normal(size=d),
        delta_bias=rng.uniform(-3.0, 0.5, d) + np.log(dt_scale),
    )
    return p


def _inputs(seed, b, d, L, ndir):
    rng = np.random.default_rng(seed)
    u = rng.normal(size=(b, d, L))
    z = rng.normal(size=(b, d, L))
    g = rng.normal(size=(b, d, L))
    dirs = [_case(rng, b, d, L) for _ in range(ndir)]
    return u, z, g, dirs


def _fwd(u, z, dirs, softplus=True, reverse=False):
    if len(dirs) == 1:
        p = dirs[0]
        return oracle.sscan_fwd(u, p["delta"], p["A"], p["B"], p["C"], p.get("D"), z, p.get("delta_bias"),
                                softplus=softplus, reverse=reverse)
    return oracle.sscan_bidir(u, z, dirs[0], dirs[1], softplus=softplus)


def _loss(u, z, g, dirs, softplus, reverse):
    return float(np.sum(g * _fwd(u, z, dirs, softplus, reverse)))


# --- G1: central finite differences of the forward oracle --------------------------------------

@pytest.mark.parametrize("ndir,reverse,softplus,gate", [
    (1, False, True, True), (1, True, True, True), (1, False, False, False), (2, False, True, True)])
def test_g1_gradients_match_central_differences(ndir, reverse, softplus, gate):
    """Each gradient entry against (L(x + h) - L(x - h)) / 2h of the forward oracle.
    Catches any wrong term, sign or index in the derivation (a dropped decay of the
    adjoint, softplus' missing, h_t used where h_{t-1} belongs, ...)."""
    b, d, L = 2, 3, 9
    u, z, g, dirs = _inputs(300 + 10 * ndir + reverse + 2 * softplus, b, d, L, ndir)
    if not softplus:
        for p in dirs:
            p["delta"] = np.abs(p["delta"]) + 0.05
            p["delta_bias"] = np.zeros(d)
    if not gate:
        z = None
    got = oracle.sscan_bwd(u, z, g, dirs, softplus=softplus, reverse=reverse)
    rng = np.random.default_rng(7)
    h = 1e-5

    def fd(mutate):
        plus, minus = mutate(h), mutate(-h)
        return (_loss(*plus, softplus, reverse) - _loss(*minus, softplus, reverse)) / (2 * h)

    def pick(shape, k=6):
        return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(k)]

    checks = []
    for idx in pick(u.shape):
        def mu(e, idx=idx):
            uu = u.copy()
            uu[idx] += e
            return uu, z, g, dirs
        checks.append(("du", idx, got["du"][idx], fd(mu)))
    if z is not None:
        for idx in pick(z.shape):
            def mz(e, idx=idx):
                zz = z.copy()
                zz[idx] += e
                return u, zz, g, dirs
            checks.append(("dz", idx, got["dz"][idx], fd(mz)))
    keys = {"ddelta": "delta", "ddelta_bias": "delta_bias", "dA": "A", "dB": "B", "dC": "C", "dD": "D"}
    for k in range(ndir):
        for gname, pname in keys.items():
            for idx in pick(dirs[k][pname].shape, 4):
                def mp(e, k=k, pname=pname, idx=idx):
                    nd = [dict(p) for p in dirs]
                    arr = nd[k][pname].copy()
                    arr[idx] += e
                    nd[k][pname] = arr
                    return u, z, g, nd
                checks.append((f"dir{k}.{gname}", idx, got["dirs"][k][gname][idx], fd(mp)))
    for name, idx, val, ref in checks:
        assert abs(val - ref) <= 1e-6 * (1.0 + abs(ref)), (name, idx, val, ref)


# --- G2: reverse-mode differentiation by PyTorch through a plain recurrence ---------------------

def _torch_forward(u, z, dirs, softplus, reverse_single):
    """Token-by-token fp64 recurrence in torch ops (the forward definition)."""
    b, d, L = u.shape
    y = torch.zeros_like(u)
    for k, p in enumerate(dirs):
        rev = reverse_single if len(dirs) == 1 else (k == 1)
        x = p["delta"] + p["delta_bias"][None, :, None]
        dt = torch.nn.functional.softplus(x) if softplus else x
        h = torch.zeros(b, d, p["A"].shape[1], dtype=torch.float64)
        ys = [None] * L
        for s in range(L):
            t = L - 1 - s if rev else s
            a = torch.exp(dt[:, :, t, None] * p["A"][None])
            h = a * h + (dt[:, :, t] * u[:, :, t])[..., None] * p["B"][:, None, :, t]
            ys[t] = (h * p["C"][:, None, :, t]).sum(-1) + p["D"][None] * u[:, :, t]
        y = y + torch.stack(ys, -1)
    return y * torch.nn.functional.silu(z) if z is not None else y


@pytest.mark.parametrize("ndir,reverse", [(1, False), (1, True), (2, False)])
def test_g2_gradients_match_autograd(ndir, reverse):
    b, d, L = 2, 4, 13
    u, z, g, dirs = _inputs(400 + 10 * ndir + reverse, b, d, L, ndir)
    got = oracle.sscan_bwd(u, z, g, dirs, reverse=reverse)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    ut, zt = T(u), T(z)
    dts = [{k: T(v) for k, v in p.items()} for p in dirs]
    out = _torch_forward(ut, zt, dts, True, reverse)
    (out * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(got["du"], ut.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dz"], zt.grad.numpy(), rtol=1e-10, atol=1e-12)
    keys = {"ddelta": "delta", "ddelta_bias": "delta_bias", "dA": "A", "dB": "B", "dC": "C", "dD": "D"}
    for k in range(ndir):
        for gname, pname in keys.items():
            ref = dts[k][pname].grad.numpy()
            np.testing.assert_allclose(got["dirs"][k][gname], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max(),
                                       err_msg=f"dir{k}.{gname}")


# --- G3: reverse direction = flip of the forward direction (Reproducing Vision Mamba page,
#         section 3.2) --------------------------------------------------------------------------

def test_g3_reverse_gradients_are_flipped_forward_gradients():
    b, d, L = 2, 3, 11
    u, z, g, dirs = _inputs(500, b, d, L, 1)
    p = dirs[0]
    rev = oracle.sscan_bwd(u, z, g, [p], reverse=True)
    fl = lambda a: np.ascontiguousarray(a[..., ::-1])
    pf = dict(p, delta=fl(p["delta"]), B=fl(p["B"]), C=fl(p["C"]))
    fwd = oracle.sscan_bwd(fl(u), fl(z), fl(g), [pf])
    np.testing.assert_allclose(rev["du"], fl(fwd["du"]), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rev["dz"], fl(fwd["dz"]), rtol=1e-12, atol=1e-13)
    for name in ("ddelta", "dB", "dC"):
        np.testing.assert_allclose(rev["dirs"][0][name], fl(fwd["dirs"][0][name]), rtol=1e-12, atol=1e-13)
    for name in ("ddelta_bias", "dA", "dD"):
        np.testing.assert_allclose(rev["dirs"][0][name], fwd["dirs"][0][name], rtol=1e-12, atol=1e-13)


def test_optional_inputs_absent_and_thread_invariance():
    b, d, L = 3, 5, 7
    u, z, g, dirs = _inputs(600, b, d, L, 1)
    p = dict(dirs[0])
    p.pop("D")
    p.pop("delta_bias")
    one = oracle.sscan_bwd(u, None, g, [p], nthreads=1)
    many = oracle.sscan_bwd(u, None, g, [p], nthreads=4)
    assert one["dz"] is None and one["dirs"][0]["dD"] is None and one["dirs"][0]["ddelta_bias"] is None
    for k in ("ddelta", "dA", "dB", "dC"):
        np.testing.assert_allclose(one["dirs"][0][k], many["dirs"][0][k], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(one["du"], many["du"], rtol=1e-13, atol=1e-14)


# --- G4: state I/O (the backward of the forward with an entry state h0 and a final
#         state h_last: Hand-written simplified Mamba2 page, section 5.2; a learned
#         initial state, Samba page, section 3.2) ------------------------------------------------

def _state_loss(u, z, g, p, h0, gh, reverse):
    out, hl = oracle.sscan_fwd(u, p["delta"], p["A"], p["B"], p["C"], p["D"], z, p["delta_bias"], reverse=reverse,
                               h0=h0, return_last_state=True)
    return float(np.sum(g * out) + np.sum(gh * hl))


@pytest.mark.parametrize("reverse", [False, True])
def test_g4_state_gradients_match_central_differences(reverse):
    """dh0 (and the gradients of u, delta, A, C with an entry state and a gradient on
    the final state) against central differences of the forward oracle's
    sum(g * out) + sum(gh * h_last)."""
    b, d, L = 2, 3, 8
    u, z, g, dirs = _inputs(700 + reverse, b, d, L, 1)
    p = dirs[0]
    rng = np.random.default_rng(701)
    h0 = rng.normal(size=(b, d, 16))
    gh = rng.normal(size=(b, d, 16))
    got = oracle.sscan_bwd(u, z, g, [p], reverse=reverse, h0=h0, dh_last=gh, return_dh0=True)
    h = 1e-5
    checks = []
    for idx in [(0, 0, 0), (1, 2, 15), (0, 1, 7), (1, 0, 3)]:
        hp, hm = h0.copy(), h0.copy()
        hp[idx] += h
        hm[idx] -= h
        ref = (_state_loss(u, z, g, p, hp, gh, reverse) - _state_loss(u, z, g, p, hm, gh, reverse)) / (2 * h)
        checks.append(("dh0", got["dh0"][idx], ref))
    for name, key, idx in [("du", None, (1, 1, 0)), ("ddelta", "delta", (0, 2, L - 1)), ("dA", "A", (1, 4)),
                           ("dC", "C", (1, 9, 0))]:
        def mut(e):
            if key is None:
                uu = u.copy()
                uu[idx] += e
                return uu, p
            q = dict(p)
            arr = q[key].copy()
            arr[idx] += e
            q[key] = arr
            return u, q
        (up, pp), (um, pm) = mut(h), mut(-h)
        ref = (_state_loss(up, z, g, pp, h0, gh, reverse) - _state_loss(um, z, g, pm, h0, gh, reverse)) / (2 * h)
        val = got["du"][idx] if key is None else got["dirs"][0]["d" + key][idx]
        checks.append((name, val, ref))
    for name, val, ref in checks:
        assert abs(val - ref) <= 1e-6 * (1.0 + abs(ref)), (name, val, ref)


def test_g4_state_gradients_match_autograd():
    """PyTorch's reverse mode through the plain recurrence started from a leaf h0,
    with a loss term on the final state."""
    b, d, L = 2, 4, 11
    u, z, g, dirs = _inputs(720, b, d, L, 1)
    p = dirs[0]
    rng = np.random.default_rng(721)
    h0 = rng.normal(size=(b, d, 16))
    gh = rng.normal(size=(b, d, 16))
    got = oracle.sscan_bwd(u, z, g, [p], h0=h0, dh_last=gh, return_dh0=True)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    ut, h0t = T(u), T(h0)
    pt = {k: T(v) for k, v in p.items()}
    x = pt["delta"] + pt["delta_bias"][None, :, None]
    dt = torch.nn.functional.softplus(x)
    h = h0t
    ys = []
    for t in range(L):
        h = torch.exp(dt[:, :, t, None] * pt["A"][None]) * h + (dt[:, :, t] * ut[:, :, t])[..., None] * pt["B"][:, None, :, t]
        ys.append((h * pt["C"][:, None, :, t]).sum(-1) + pt["D"][None] * ut[:, :, t])
    out = torch.stack(ys, -1) * torch.nn.functional.silu(torch.tensor(z))
    ((out * torch.tensor(g)).sum() + (h * torch.tensor(gh)).sum()).backward()
    np.testing.assert_allclose(got["dh0"], h0t.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["du"], ut.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dirs"][0]["dA"], pt["A"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dirs"][0]["ddelta"], pt["delta"].grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("reverse", [False, True])
def test_g4_backward_of_pieces_equals_backward_of_the_whole(reverse):
    """A sequence cut in two pieces, the state handed from the first to the second
    (forward) and dh0 of the second handed back as dh_last of the first (backward):
    the pieces' gradients, put together, are the whole sequence's."""
    b, d, L, m = 2, 3, 17, 6
    u, z, g, dirs = _inputs(740 + reverse, b, d, L, 1)
    p = dirs[0]
    whole = oracle.sscan_bwd(u, z, g, [p], reverse=reverse)
    first, second = (slice(m, L), slice(0, m)) if reverse else (slice(0, m), slice(m, L))
    cut = lambda a, s: np.ascontiguousarray(a[..., s])
    pc = lambda s: dict(p, delta=cut(p["delta"], s), B=cut(p["B"], s), C=cut(p["C"], s))
    _, hmid = oracle.sscan_fwd(cut(u, first), pc(first)["delta"], p["A"], pc(first)["B"], pc(first)["C"], p["D"],
                               cut(z, first), p["delta_bias"], reverse=reverse, return_last_state=True)
    g2 = oracle.sscan_bwd(cut(u, second), cut(z, second), cut(g, second), [pc(second)], reverse=reverse, h0=hmid,
                          return_dh0=True)
    g1 = oracle.sscan_bwd(cut(u, first), cut(z, first), cut(g, first), [pc(first)], reverse=reverse,
                          dh_last=g2["dh0"])
    join = lambda a1, a2: np.concatenate([a1, a2] if not reverse else [a2, a1], axis=-1)
    np.testing.assert_allclose(join(g1["du"], g2["du"]), whole["du"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(join(g1["dz"], g2["dz"]), whole["dz"], rtol=1e-11, atol=1e-12)
    for k in ("ddelta", "dB", "dC"):
        np.testing.assert_allclose(join(g1["dirs"][0][k], g2["dirs"][0][k]), whole["dirs"][0][k], rtol=1e-11,
                                   atol=1e-12, err_msg=k)
    for k in ("dA", "dD", "ddelta_bias"):
        np.testing.assert_allclose(g1["dirs"][0][k] + g2["dirs"][0][k], whole["dirs"][0][k], rtol=1e-11, atol=1e-12,
                                   err_msg=k)


def test_g4_empty_sequence_passes_the_state_gradient_through():
    b, d = 2, 3
    rng = np.random.default_rng(760)
    gh = rng.normal(size=(b, d, 16))
    u, z, g, dirs = _inputs(761, b, d, 0, 1)
    got = oracle.sscan_bwd(u, z, g, dirs, dh_last=gh, h0=rng.normal(size=(b, d, 16)), return_dh0=True)
    np.testing.assert_array_equal(got["dh0"], gh)
