"""Pins of the fp64 oracle against what the pages and the mathematics fix.

No HIP code is involved.  Each test names the passage it follows and the kind of
mistake in the oracle it would catch.
"""
import math

import numpy as np
import pytest

from oracle import brute


def _case(rng, b, d, L, N, softplus=True, positive_dt=False):
    """Random fp64 inputs; A differs per (d, n) so a transposed A is caught."""
    p = dict(
        delta=rng.normal(0.0, 0.5, (b, d, L)) + (1.0 if positive_dt else 0.0),
        A=-np.exp(rng.uniform(-1.0, 1.5, (d, N))),
        B=rng.normal(size=(b, N, L)),
        C=rng.normal(size=(b, N, L)),
        D=rng.normal(size=d),
        delta_bias=rng.uniform(-3.0, 0.5, d),
    )
    u = rng.normal(size=(b, d, L))
    z = rng.normal(size=(b, d, L))
    return u, z, p


def _fwd(o, u, p, z=None, **kw):
    return o.sscan_fwd(u, p["delta"], p["A"], p["B"], p["C"], p.get("D"), z, p.get("delta_bias"), **kw)


def _softplus_lib(x):
    return np.logaddexp(0.0, x)


def _silu_lib(x):
    return x / (1.0 + np.exp(-x))


# --- P1: LTI convolution (Hand-written simplified Mamba2 page, sections 2.3, 4.3, 4.5) ---------

@pytest.mark.parametrize("reverse", [False, True])
def test_p1_lti_matches_convolution_kernel(oracle_lib, reverse):
    """Constant dt, B, C over t: output = (K * u)_t + D u_t with
    K_k = sum_n C_n Abar_n^k dt B_n.  Catches wrong exp sign, wrong recurrence
    order, a missing dt on B, a readout of the old state."""
    rng = np.random.default_rng(11)
    b, d, L, N = 2, 3, 40, 6
    u, z, p = _case(rng, b, d, L, N)
    dt_c = rng.uniform(0.05, 0.4, d)
    Bc = rng.normal(size=(b, N))
    Cc = rng.normal(size=(b, N))
    p["delta"] = np.broadcast_to(dt_c[None, :, None], (b, d, L)).copy()
    p["B"] = np.broadcast_to(Bc[:, :, None], (b, N, L)).copy()
    p["C"] = np.broadcast_to(Cc[:, :, None], (b, N, L)).copy()
    p["delta_bias"] = None
    y = _fwd(oracle_lib, u, p, softplus=False, reverse=reverse)
    ref = np.empty_like(y)
    for bi in range(b):
        for di in range(d):
            Abar = np.exp(dt_c[di] * p["A"][di])
            K = np.array([np.sum(Cc[bi] * Abar ** k * dt_c[di] * Bc[bi]) for k in range(L)])
            if not reverse:
                conv = np.convolve(u[bi, di], K)[:L]
            else:
                conv = np.convolve(u[bi, di][::-1], K)[:L][::-1]
            ref[bi, di] = conv + p["D"][di] * u[bi, di]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_p1_constant_input_geometric_closed_form(oracle_lib):
    """u == const: y_t = sum_n C_n dt B_n u (1 - Abar_n^{t+1}) / (1 - Abar_n) + D u."""
    rng = np.random.default_rng(12)
    d, L, N = 4, 64, 16
    dt_c = rng.uniform(0.01, 0.3, d)
    A = -np.arange(1, N + 1, dtype=np.float64)[None, :] * rng.uniform(0.5, 2.0, (d, 1))
    Bc, Cc = rng.normal(size=N), rng.normal(size=N)
    D = rng.normal(size=d)
    uval = 0.7
    y = oracle_lib.sscan_fwd(np.full((1, d, L), uval), np.broadcast_to(dt_c[None, :, None], (1, d, L)), A,
                             np.broadcast_to(Bc[None, :, None], (1, N, L)), np.broadcast_to(Cc[None, :, None], (1, N, L)),
                             D, None, None, softplus=False)
    t = np.arange(L)
    for di in range(d):
        Ab = np.exp(dt_c[di] * A[di])
        ref = sum(Cc[n] * dt_c[di] * Bc[n] * uval * (1 - Ab[n] ** (t + 1)) / (1 - Ab[n]) for n in range(N))
        ref = ref + D[di] * uval
        np.testing.assert_allclose(y[0, di], ref, rtol=1e-12, atol=1e-13)


# --- P2: L = 1 closed form (same page, section 2.2 and the gate of section 4.4) ---------------

def test_p2_len1_closed_form_fwd(oracle_lib):
    """out_0 = (dt_0 sum_n C_n B_n + D) u_0 silu(z_0); A plays no role.  Catches a
    bias added after softplus, a missing D, the gate applied to only part of y."""
    rng = np.random.default_rng(21)
    b, d, N = 3, 5, 16
    u, z, p = _case(rng, b, d, 1, N)
    out = _fwd(oracle_lib, u, p, z=z)
    dt = _softplus_lib(p["delta"][:, :, 0] + p["delta_bias"][None, :])
    cb = np.einsum("bn,bn->b", p["C"][:, :, 0], p["B"][:, :, 0])
    ref = (dt * cb[:, None] + p["D"][None, :]) * u[:, :, 0] * _silu_lib(z[:, :, 0])
    np.testing.assert_allclose(out[:, :, 0], ref, rtol=1e-14, atol=1e-15)


def test_p2_len1_closed_form_bidir(oracle_lib):
    rng = np.random.default_rng(22)
    b, d, N = 2, 4, 16
    u, z, pf = _case(rng, b, d, 1, N)
    _, _, pr = _case(rng, b, d, 1, N)
    out = oracle_lib.sscan_bidir(u, z, pf, pr)
    ref = 0.0
    for p in (pf, pr):
        dt = _softplus_lib(p["delta"][:, :, 0] + p["delta_bias"][None, :])
        cb = np.einsum("bn,bn->b", p["C"][:, :, 0], p["B"][:, :, 0])
        ref = ref + dt * cb[:, None] + p["D"][None, :]
    ref = ref * u[:, :, 0] * _silu_lib(z[:, :, 0])
    np.testing.assert_allclose(out[:, :, 0], ref, rtol=1e-14, atol=1e-15)


# --- P3: dt -> 0 leaves the state unchanged (Mamba2 page, section 2.4; Samba page's masked
#         tokens that skip the scan) -----------------------------------------------------------

def test_p3i_zero_step_gives_skip_only(oracle_lib):
    rng = np.random.default_rng(31)
    u, z, p = _case(rng, 2, 3, 17, 16)
    p["delta"] = np.zeros_like(p["delta"])
    p["delta_bias"] = None
    out = _fwd(oracle_lib, u, p, z=z, softplus=False)
    np.testing.assert_allclose(out, p["D"][None, :, None] * u * _silu_lib(z), rtol=1e-15, atol=0)


def test_p3ii_masked_tokens_are_bypassed(oracle_lib):
    """dt = 0 on a token set M: outputs outside M equal those of the sequence with
    M deleted, and on M the readout sees the state left by the last kept token."""
    rng = np.random.default_rng(32)
    b, d, L, N = 2, 3, 30, 16
    u, z, p = _case(rng, b, d, L, N, positive_dt=True)
    p["delta_bias"] = None
    p["delta"] = np.abs(p["delta"]) + 0.05
    M = np.zeros(L, bool)
    M[[0, 3, 4, 5, 11, 20, 29]] = True
    p["delta"][:, :, M] = 0.0
    full = _fwd(oracle_lib, u, p, softplus=False)
    keep = ~M
    pk = dict(p, delta=p["delta"][:, :, keep], B=p["B"][:, :, keep], C=p["C"][:, :, keep])
    comp = _fwd(oracle_lib, u[:, :, keep], pk, softplus=False)
    np.testing.assert_allclose(full[:, :, keep], comp, rtol=1e-13, atol=1e-14)
    for t in np.nonzero(M)[0]:
        kept_before = int(keep[:t].sum())
        if kept_before == 0:
            h = np.zeros((b, d, N))
        else:
            pre = dict(pk, delta=pk["delta"][:, :, :kept_before], B=pk["B"][:, :, :kept_before],
                       C=pk["C"][:, :, :kept_before])
            _, h = _fwd(oracle_lib, u[:, :, keep][:, :, :kept_before], pre, softplus=False, return_last_state=True)
        ref = np.einsum("bdn,bn->bd", h, p["C"][:, :, t]) + p["D"][None, :] * u[:, :, t]
        np.testing.assert_allclose(full[:, :, t], ref, rtol=1e-13, atol=1e-14)


def test_p3iii_softplus_of_very_negative_is_the_zero_limit(oracle_lib):
    rng = np.random.default_rng(33)
    u, z, p = _case(rng, 1, 4, 25, 16)
    p["delta"] = np.full_like(p["delta"], -60.0)
    p["delta_bias"] = np.zeros(4)
    out = _fwd(oracle_lib, u, p, z=z, softplus=True)
    ref = p["D"][None, :, None] * u * _silu_lib(z)
    np.testing.assert_allclose(out, ref, rtol=1e-15, atol=0)


# --- P4: reverse = flip . forward . flip (Reproducing Vision Mamba page, section 3.2) ----------

def test_p4_reverse_is_flipped_forward(oracle_lib):
    rng = np.random.default_rng(41)
    u, z, p = _case(rng, 2, 3, 37, 16)
    rev = _fwd(oracle_lib, u, p, z=z, reverse=True)
    fl = lambda a: np.ascontiguousarray(a[..., ::-1])
    pf = dict(p, delta=fl(p["delta"]), B=fl(p["B"]), C=fl(p["C"]))
    fwd_of_flipped = _fwd(oracle_lib, fl(u), pf, z=fl(z), reverse=False)
    np.testing.assert_array_equal(rev, fl(fwd_of_flipped))
    assert not np.allclose(rev, _fwd(oracle_lib, u, p, z=z, reverse=False))


# --- P5: brute force (materialised dual form, Mamba2 page section 3.1) -------------------------

@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("mode", ["fwd", "rev", "bidir"])
def test_p5_oracle_matches_materialised_form(oracle_lib, softplus, mode):
    rng = np.random.default_rng(51 + (mode == "rev") * 7 + (mode == "bidir") * 13 + softplus)
    b, d, L, N = 2, 3, 23, 5
    u, z, pf = _case(rng, b, d, L, N)
    _, _, pr = _case(rng, b, d, L, N)
    if not softplus:
        pf["delta"] = np.abs(pf["delta"]) * 0.3
        pr["delta"] = np.abs(pr["delta"]) * 0.3
        pf["delta_bias"] = pr["delta_bias"] = None
    if mode == "bidir":
        got = oracle_lib.sscan_bidir(u, z, pf, pr, softplus=softplus)
        ref = brute.brute(u, z, [pf, pr], softplus=softplus)
    else:
        got = _fwd(oracle_lib, u, pf, z=z, softplus=softplus, reverse=(mode == "rev"))
        ref = brute.brute(u, z, [pf], softplus=softplus, reverse_single=(mode == "rev"))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("mode", ["fwd", "rev", "bidir"])
def test_p5_oracle_certified_by_mpmath(oracle_lib, mode):
    """50-digit evaluation of the materialised form on tiny inputs: the fp64
    oracle must agree to ~1e-14 relative."""
    rng = np.random.default_rng(61 + len(mode))
    b, d, L, N = 1, 2, 7, 3
    u, z, pf = _case(rng, b, d, L, N)
    _, _, pr = _case(rng, b, d, L, N)
    if mode == "bidir":
        got = oracle_lib.sscan_bidir(u, z, pf, pr)
        ref = brute.brute_mp(u, z, [pf, pr])
    else:
        got = _fwd(oracle_lib, u, pf, z=z, reverse=(mode == "rev"))
        ref = brute.brute_mp(u, z, [pf], reverse_single=(mode == "rev"))
    ref = np.array([[[float(v) for v in row] for row in plane] for plane in ref])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14 * np.abs(ref).max())


# --- P6: A = 0 turns the scan into a prefix sum ---------------------------------------------------

def test_p6_zero_A_is_prefix_sum(oracle_lib):
    rng = np.random.default_rng(71)
    b, d, L, N = 2, 3, 50, 16
    u, z, p = _case(rng, b, d, L, N)
    p["A"] = np.zeros((d, N))
    y = _fwd(oracle_lib, u, p)
    dt = _softplus_lib(p["delta"] + p["delta_bias"][None, :, None])
    w = dt[:, :, None, :] * p["B"][:, None, :, :] * u[:, :, None, :]  # [b,d,N,L]
    h = np.cumsum(w, axis=-1)
    ref = np.einsum("bdnt,bnt->bdt", h, p["C"]) + p["D"][None, :, None] * u
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# --- P7: linearity (the recurrence and readout of section 2.2 are linear in u, B, C) ------------

def test_p7_linearity(oracle_lib):
    rng = np.random.default_rng(81)
    u1, _, p = _case(rng, 2, 3, 31, 16)
    u2 = rng.normal(size=u1.shape)
    a, c = 1.7, -0.4
    y = lambda u, q: _fwd(oracle_lib, u, q)
    scale = np.abs(y(u1, p)).max()
    np.testing.assert_allclose(y(a * u1 + c * u2, p), a * y(u1, p) + c * y(u2, p), rtol=1e-11, atol=1e-12 * scale)
    noD = dict(p, D=None)
    C2 = rng.normal(size=p["C"].shape)
    np.testing.assert_allclose(y(u1, dict(noD, C=a * p["C"] + c * C2)),
                               a * y(u1, noD) + c * y(u1, dict(noD, C=C2)), rtol=1e-11, atol=1e-12 * scale)
    B2 = rng.normal(size=p["B"].shape)
    np.testing.assert_allclose(y(u1, dict(noD, B=a * p["B"] + c * B2)),
                               a * y(u1, noD) + c * y(u1, dict(noD, B=B2)), rtol=1e-11, atol=1e-12 * scale)


# --- P8: bidirectional composition: the sum precedes the single gate (Vim page, section 3.1) ----

def test_p8_bidir_sum_then_gate(oracle_lib):
    rng = np.random.default_rng(91)
    u, z, pf = _case(rng, 2, 3, 19, 16)
    _, _, pr = _case(rng, 2, 3, 19, 16)
    got = oracle_lib.sscan_bidir(u, z, pf, pr)
    yf = _fwd(oracle_lib, u, pf)
    yr = _fwd(oracle_lib, u, pr, reverse=True)
    np.testing.assert_allclose(got, (yf + yr) * _silu_lib(z), rtol=1e-13, atol=1e-14)


# --- P9: determinism (Vim page, section 1.2: two runs must agree exactly) -----------------------

def test_p9_deterministic_and_thread_invariant(oracle_lib):
    rng = np.random.default_rng(95)
    u, z, p = _case(rng, 3, 5, 40, 16)
    a = _fwd(oracle_lib, u, p, z=z, nthreads=1)
    b = _fwd(oracle_lib, u, p, z=z, nthreads=1)
    c = _fwd(oracle_lib, u, p, z=z, nthreads=4)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


# --- P10: memoryless limit (strongly negative A: Abar ~ 0) -------------------------------------

def test_p10_memoryless_limit(oracle_lib):
    rng = np.random.default_rng(101)
    u, z, p = _case(rng, 2, 3, 21, 16)
    p["A"] = np.full_like(p["A"], -1e6)
    p["delta_bias"] = np.full(3, 2.0)  # dt >= softplus(2 - 2.5) > 0.4: Abar < exp(-4e5)
    y = _fwd(oracle_lib, u, p)
    dt = _softplus_lib(p["delta"] + p["delta_bias"][None, :, None])
    cb = np.einsum("bnt,bnt->bt", p["C"], p["B"])
    ref = dt * cb[:, None, :] * u + p["D"][None, :, None] * u
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


# --- P11: the state is carried across chunks (Mamba2 page section 3.2 / the remark after 4.4;
#          YOLO26 page section 5.1: segments pass their hidden state on) ----------------------

@pytest.mark.parametrize("reverse", [False, True])
def test_p11_chunk_carry_invariance(oracle_lib, reverse):
    rng = np.random.default_rng(111)
    b, d, L, N = 2, 3, 75, 16
    u, z, p = _case(rng, b, d, L, N)
    full = _fwd(oracle_lib, u, p, reverse=reverse)

    def chunked(size, carry):
        out = np.empty_like(full)
        h = None
        bounds = list(range(0, L, size))
        if reverse:
            bounds = bounds[::-1]
        for s in bounds:
            e = min(L, s + size)
            q = dict(p, delta=p["delta"][:, :, s:e], B=p["B"][:, :, s:e], C=p["C"][:, :, s:e])
            y, hl = _fwd(oracle_lib, u[:, :, s:e], q, reverse=reverse, h0=h if carry else None,
                         return_last_state=True)
            out[:, :, s:e] = y
            h = hl
        return out

    for size in (1, 7, 32, 64, L):
        np.testing.assert_array_equal(chunked(size, True), full)
    reset = chunked(32, False)
    assert np.abs(reset - full).max() > 1e-3 * np.abs(full).max()


# --- P12: entry state and final state (Mamba2 page, section 5.2: recurrent inference carries
#          the fixed-size state from one call to the next; YOLO26 page section 5.1) -------------

@pytest.mark.parametrize("reverse", [False, True])
def test_p12_entry_and_last_state_match_materialised_form(oracle_lib, reverse):
    """Outputs with an entry state h0 and the returned last state against the
    weighted-sum forms of ``brute`` (no recurrence).  Catches h0 read in the wrong
    layout ([b, d, N] with N fastest), decayed by the wrong prefix, or a last
    state taken one token early."""
    rng = np.random.default_rng(121)
    b, d, L, N = 2, 3, 23, 16
    u, z, p = _case(rng, b, d, L, N)
    h0 = rng.normal(size=(b, d, N))
    out, hl = _fwd(oracle_lib, u, p, z=z, reverse=reverse, h0=h0, return_last_state=True)
    ref = brute.brute_dir(u, reverse=reverse, h0=h0, **p) * _silu_lib(z)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())
    ref_h = brute.brute_last_state(u, p["delta"], p["A"], p["B"], p["delta_bias"], reverse=reverse, h0=h0)
    np.testing.assert_allclose(hl, ref_h, rtol=1e-11, atol=1e-12 * np.abs(ref_h).max())


def test_p12_len1_step_closed_form(oracle_lib):
    """One token from state h0 (the single-step decode): h_n = exp(dt A_n) h0_n +
    dt B_n u, out = (sum_n C_n h_n + D u) silu(z).  Catches A transposed, the
    decay applied to the input term, or the old state read out."""
    rng = np.random.default_rng(122)
    b, d, N = 3, 4, 16
    u, z, p = _case(rng, b, d, 1, N)
    h0 = rng.normal(size=(b, d, N))
    out, hl = _fwd(oracle_lib, u, p, z=z, h0=h0, return_last_state=True)
    dt = _softplus_lib(p["delta"][:, :, 0] + p["delta_bias"][None, :])  # [b, d]
    h = np.exp(dt[..., None] * p["A"][None]) * h0 + dt[..., None] * p["B"][:, None, :, 0] * u[:, :, :1]
    ref = (np.einsum("bn,bdn->bd", p["C"][:, :, 0], h) + p["D"][None] * u[:, :, 0]) * _silu_lib(z[:, :, 0])
    np.testing.assert_allclose(hl, h, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out[:, :, 0], ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("reverse", [False, True])
def test_p12_no_tokens_hand_the_state_through(oracle_lib, reverse):
    """A piece of a stream with no tokens applies the recurrence zero times, so the
    final state is the entry state (zeros without one) and the output is empty.
    Catches a final state left unwritten when the sequence is empty."""
    rng = np.random.default_rng(123)
    b, d, N = 2, 5, 16
    u, z, p = _case(rng, b, d, 0, N)
    h0 = rng.normal(size=(b, d, N))
    out, hl = _fwd(oracle_lib, u, p, z=z, reverse=reverse, h0=h0, return_last_state=True)
    assert out.shape == (b, d, 0)
    np.testing.assert_array_equal(hl, h0)
    _, hl0 = _fwd(oracle_lib, u, p, z=z, reverse=reverse, return_last_state=True)
    np.testing.assert_array_equal(hl0, np.zeros((b, d, N)))


# --- scalar helpers and special values ------------------------------------------------------------

@pytest.mark.parametrize("x", [-700.0, -60.0, -20.0, -9.2, -3.0, -1e-8, 0.0, 1e-8, 2.5, 20.0, 60.0, 700.0])
def test_softplus_and_silu_against_mpmath(oracle_lib, x):
    import mpmath as mp
    mp.mp.dps = 40
    sp = mp.log1p(mp.exp(mp.mpf(x)))
    assert oracle_lib.softplus(x) == pytest.approx(float(sp), rel=4e-16, abs=0.0)
    si = mp.mpf(x) / (1 + mp.exp(-mp.mpf(x)))
    assert oracle_lib.silu(x) == pytest.approx(float(si), rel=4e-16, abs=1e-300)


def test_nan_propagates_along_scan_direction(oracle_lib):
    rng = np.random.default_rng(121)
    u, z, p = _case(rng, 2, 3, 20, 16)
    u = u.copy()
    u[1, 2, 9] = math.nan
    fwd = _fwd(oracle_lib, u, p, z=z)
    assert np.isnan(fwd[1, 2, 9:]).all() and np.isfinite(fwd[1, 2, :9]).all()
    rev = _fwd(oracle_lib, u, p, z=z, reverse=True)
    assert np.isnan(rev[1, 2, :10]).all() and np.isfinite(rev[1, 2, 10:]).all()
    mask = np.ones(fwd.shape, bool)
    mask[1, 2] = False
    assert np.isfinite(fwd[mask]).all() and np.isfinite(rev[mask]).all()


def test_empty_inputs_are_a_no_op(oracle_lib):
    out = oracle_lib.sscan_fwd(np.zeros((2, 3, 0)), np.zeros((2, 3, 0)), -np.ones((3, 16)), np.zeros((2, 16, 0)),
                               np.zeros((2, 16, 0)))
    assert out.shape == (2, 3, 0)
