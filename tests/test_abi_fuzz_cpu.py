"""Randomised checks of the argument validation of sscan_fwd and sscan_bidir (no GPU).

A valid layout of fake, disjoint device addresses is mutated at random: pointers
set to NULL or moved off their alignment, the output placed over an input, the
workspace shrunk, moved or placed over the output, sizes made negative or zero,
dtype codes and dstate made unsupported.  A model of the rules the header states
lists every rule the mutated call breaks, and the validator must return SSCAN_OK
exactly when that list is empty, else one of the listed codes (the order in which
the library checks them is not part of the contract).  Pointers are never
dereferenced.
"""
import ctypes

from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from selective_state_space_sscan_amd import sscan
from test_abi_cpu import EALIAS, EALIGN, ENULL, ESHAPE, EUNSUP, EWS, OK, Fake, lib  # noqa: F401

IO_PTRS = ("u", "z", "y")
DIR_PTRS = ("delta", "bias", "A", "B", "C", "D")
REQUIRED = {"u", "y", "delta", "A", "B", "C"}


def esz(code):
    return 2 if code == 1 else 4


def layout(b, d, L, io, bc, ndir, ws_need):
    """Disjoint fake buffers of the right sizes for a call of these sizes."""
    f = Fake()
    ie, be = esz(io), esz(bc)
    n_io, n_bc = max(b * d * L, 1), max(b * 16 * L, 1)
    a = {k: f(n_io * ie) for k in IO_PTRS}
    for k in range(ndir):
        a.update({f"{k}.delta": f(n_io * ie), f"{k}.bias": f(max(d, 1) * 4), f"{k}.A": f(max(d, 1) * 64),
                  f"{k}.B": f(n_bc * be), f"{k}.C": f(n_bc * be), f"{k}.D": f(max(d, 1) * 4)})
    a["ws"] = f(max(ws_need, 1))
    a["ws_bytes"] = ws_need
    return a


def sizes_of(b, d, L, io, bc):
    ie, be = esz(io), esz(bc)
    return {"u": b * d * L * ie, "z": b * d * L * ie, "y": b * d * L * ie, "delta": b * d * L * ie,
            "bias": d * 4, "A": d * 64, "B": b * 16 * L * be, "C": b * 16 * L * be, "D": d * 4}


def expected(a, b, d, L, N, io, bc, ndir, ws_need):
    """Every status code whose rule the call breaks (empty: the call is valid)."""
    bad = set()
    if b < 0 or d < 0 or L < 0:
        bad.add(ESHAPE)
    if N != 16 or io not in (0, 1) or bc not in (0, 1):
        bad.add(EUNSUP)
    if bad:
        return bad
    if b == 0 or d == 0 or L == 0:
        return set()  # a valid empty call, whatever the pointers
    sz = sizes_of(b, d, L, io, bc)
    align = {"u": esz(io), "z": esz(io), "y": esz(io), "delta": esz(io), "B": esz(bc), "C": esz(bc),
             "A": 4, "bias": 4, "D": 4}
    names = list(IO_PTRS) + [f"{k}.{n}" for k in range(ndir) for n in DIR_PTRS]
    base = lambda name: name.split(".")[-1]
    for name in names:
        p = a[name]
        if p is None:
            if base(name) in REQUIRED:
                bad.add(ENULL)
            continue
        if p % align[base(name)]:
            bad.add(EALIGN)
    y = a["y"]
    if y is not None:
        y_hi = y + sz["y"]
        for name in names:
            p = a[name]
            if name == "y" or p is None:
                continue
            if p < y_hi and y < p + sz[base(name)]:
                bad.add(EALIAS)
    if ws_need > 0:
        ws = a["ws"]
        if ws is None or a["ws_bytes"] < ws_need:
            bad.add(EWS)
        elif ws % 16:
            bad.add(EALIGN)
        elif y is not None and ws < y + sz["y"] and y < ws + ws_need:
            bad.add(EALIAS)
    return bad


MUTATIONS = st.lists(st.sampled_from(["null", "misalign", "alias_y", "ws_short", "ws_null", "ws_misalign",
                                      "ws_over_y"]), max_size=3)


@st.composite
def calls(draw, ndir):
    b = draw(st.sampled_from([0, 1, 2, 3]) | st.integers(-2, -1))
    d = draw(st.sampled_from([0, 1, 64, 65, 200]))
    L = draw(st.sampled_from([0, 1, 31, 32, 197, 600, 5000]))
    N = draw(st.sampled_from([16, 16, 16, 8, 32]))
    io = draw(st.sampled_from([0, 1, 1, 2]))
    bc = draw(st.sampled_from([0, 1, 0, -1]))
    return b, d, L, N, io, bc, draw(MUTATIONS), draw(st.randoms(use_true_random=False))


def mutate(a, muts, rnd, ndir):
    names = list(IO_PTRS) + [f"{k}.{n}" for k in range(ndir) for n in DIR_PTRS]
    for m in muts:
        if m == "null":
            a[rnd.choice(names)] = None
        elif m == "misalign":
            k = rnd.choice(names)
            if a[k] is not None:
                a[k] += rnd.choice([1, 2, 4, 8])
        elif m == "alias_y":
            k = rnd.choice([n for n in names if n != "y"])
            if a[k] is not None:
                a["y"] = a[k] + rnd.choice([0, 4, 64])
        elif m == "ws_short":
            a["ws_bytes"] = max(0, a["ws_bytes"] - rnd.choice([1, 256, 1 << 20]))
        elif m == "ws_null":
            a["ws"] = None
        elif m == "ws_misalign":
            if a["ws"] is not None:
                a["ws"] += rnd.choice([4, 8, 12])
        elif m == "ws_over_y":
            if a["y"] is not None:
                a["ws"] = a["y"] + rnd.choice([0, 16, 256])


def ws_bytes_for(lib, b, d, L, N, io, bc, bidir):
    if b <= 0 or d <= 0 or L <= 0 or N != 16 or io not in (0, 1) or bc not in (0, 1):
        return 0
    return int(lib.sscan_workspace_bytes(b, d, L, N, int(bidir)))


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(calls(ndir=1))
def test_validate_fwd_matches_the_rules(lib, call):
    b, d, L, N, io, bc, muts, rnd = call
    need = ws_bytes_for(lib, b, d, L, N, io, bc, False)
    a = layout(max(b, 0), max(d, 0), max(L, 0), io if io in (0, 1) else 0, bc if bc in (0, 1) else 0, 1, need)
    mutate(a, muts, rnd, 1)
    got = lib.sscan_validate_fwd(a["u"], a["0.delta"], a["0.bias"], 1, a["0.A"], a["0.B"], a["0.C"], a["0.D"],
                                 a["z"], a["y"], b, d, L, N, 0, io, bc, a["ws"], a["ws_bytes"])
    want = expected(a, b, d, L, N, io, bc, 1, need)
    if want:
        assert got in want, (got, want, muts, (b, d, L, N, io, bc))
    else:
        assert got == OK, (got, muts, (b, d, L, N, io, bc))


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(calls(ndir=2))
def test_validate_bidir_matches_the_rules(lib, call):
    b, d, L, N, io, bc, muts, rnd = call
    need = ws_bytes_for(lib, b, d, L, N, io, bc, True)
    a = layout(max(b, 0), max(d, 0), max(L, 0), io if io in (0, 1) else 0, bc if bc in (0, 1) else 0, 2, need)
    mutate(a, muts, rnd, 2)
    dirs = [sscan.DirParams(a[f"{k}.delta"], a[f"{k}.bias"], a[f"{k}.A"], a[f"{k}.B"], a[f"{k}.C"], a[f"{k}.D"])
            for k in range(2)]
    got = lib.sscan_validate_bidir(a["u"], a["z"], a["y"], ctypes.byref(dirs[0]), ctypes.byref(dirs[1]), 1, b, d, L, N,
                                   io, bc, a["ws"], a["ws_bytes"])
    want = expected(a, b, d, L, N, io, bc, 2, need)
    if want:
        assert got in want, (got, want, muts, (b, d, L, N, io, bc))
    else:
        assert got == OK, (got, muts, (b, d, L, N, io, bc))


def test_a_shared_delta_is_allowed_in_bidir(lib):
    """The two directions may read one delta tensor (the Vim and Mamba-YOLO case)."""
    need = int(lib.sscan_workspace_bytes(2, 64, 197, 16, 1))
    a = layout(2, 64, 197, 1, 1, 2, need)
    a["1.delta"] = a["0.delta"]
    dirs = [sscan.DirParams(a[f"{k}.delta"], a[f"{k}.bias"], a[f"{k}.A"], a[f"{k}.B"], a[f"{k}.C"], a[f"{k}.D"])
            for k in range(2)]
    assert lib.sscan_validate_bidir(a["u"], a["z"], a["y"], ctypes.byref(dirs[0]), ctypes.byref(dirs[1]), 1, 2, 64, 197,
                                    16, 1, 1, a["ws"], a["ws_bytes"]) == OK


# ---- the backward (sscan_bwd): gradients as outputs ---------------------------------

BWD_IO = ("u", "z", "dout", "du", "dz")
BWD_DIR_IN = ("delta", "bias", "A", "B", "C", "D")
BWD_GRADS = ("ddelta", "dbias", "dA", "dB", "dC", "dD")


def bwd_sizes(b, d, L, io, bc):
    ie, be = esz(io), esz(bc)
    s = {k: b * d * L * ie for k in ("u", "z", "dout", "du", "dz", "delta", "ddelta")}
    s.update(bias=d * 4, dbias=d * 4, D=d * 4, dD=d * 4, A=d * 64, dA=d * 64,
             B=b * 16 * L * be, C=b * 16 * L * be, dB=b * 16 * L * be, dC=b * 16 * L * be)
    return s


def bwd_layout(b, d, L, io, bc, ws_need):
    f = Fake()
    s = bwd_sizes(max(b, 1), max(d, 1), max(L, 1), io, bc)
    a = {k: f(s[k]) for k in BWD_IO + BWD_DIR_IN + BWD_GRADS}
    a["ws"] = f(max(ws_need, 1))
    a["ws_bytes"] = ws_need
    return a


def bwd_expected(a, b, d, L, N, io, bc, ws_need):
    """Every status code whose rule (as the header states it) the call breaks."""
    bad = set()
    if b < 0 or d < 0 or L < 0:
        bad.add(ESHAPE)
    if N != 16 or io not in (0, 1) or bc not in (0, 1):
        bad.add(EUNSUP)
    if bad:
        return bad
    empty = b == 0 or d == 0 or L == 0
    sz = bwd_sizes(b, d, L, io, bc)
    ie, be = esz(io), esz(bc)
    # gradient buffers are required whenever they have elements, empty call or not
    if (sz["dA"] and a["dA"] is None) or (sz["dB"] and (a["dB"] is None or a["dC"] is None)):
        bad.add(ENULL)
    z_given = a["z"] is not None
    if not empty:
        for k in ("u", "dout", "du", "delta", "A", "B", "C", "ddelta") + (("dz",) if z_given else ()):
            if a[k] is None:
                bad.add(ENULL)
    align = dict(A=4, bias=4, D=4, dA=4, dbias=4, dD=4, dB=be, dC=be)
    if not empty:
        align.update({k: ie for k in ("u", "z", "dout", "du", "dz", "delta", "ddelta")}, B=be, C=be)
    for k, n in align.items():
        if k == "dz" and not z_given:
            continue
        if a[k] is not None and a[k] % n:
            bad.add(EALIGN)
    # outputs: the parameter gradients always; du, dz, ddelta and the workspace when not empty
    outs = ["dA", "dbias", "dD", "dB", "dC"]
    ins = []
    if not empty:
        outs += ["du", "ddelta"] + (["dz"] if z_given else [])
        ins = ["u", "z", "dout", "delta", "B", "C", "A", "bias", "D"]
    rng = {k: (a[k], a[k] + sz[k]) for k in outs + ins if a[k] is not None and sz[k] > 0}
    if not empty:
        ws = a["ws"]
        if ws is None or a["ws_bytes"] < ws_need:
            bad.add(EWS)
        elif ws % 16:
            bad.add(EALIGN)
        else:
            rng["ws"] = (ws, ws + ws_need)
            outs = outs + ["ws"]
    hit = lambda p, q: p[0] < q[1] and q[0] < p[1]
    live_outs = [k for k in outs if k in rng]
    for i, o in enumerate(live_outs):
        if any(hit(rng[o], rng[k]) for k in ins if k in rng) or any(hit(rng[o], rng[k]) for k in live_outs[i + 1:]):
            bad.add(EALIAS)
    return bad


BWD_MUTATIONS = st.lists(st.sampled_from(["null", "null_grad", "misalign", "alias_out", "ws_short", "ws_null",
                                          "ws_misalign", "ws_over_out", "no_z"]), max_size=3)


@st.composite
def bwd_calls(draw):
    b = draw(st.sampled_from([0, 1, 2]) | st.integers(-1, -1))
    d = draw(st.sampled_from([0, 1, 64, 130]))
    L = draw(st.sampled_from([0, 1, 32, 197, 3000]))
    N = draw(st.sampled_from([16, 16, 16, 8]))
    io = draw(st.sampled_from([0, 1, 1, 2]))
    bc = draw(st.sampled_from([0, 1, 0, -1]))
    return b, d, L, N, io, bc, draw(BWD_MUTATIONS), draw(st.randoms(use_true_random=False))


def bwd_mutate(a, muts, rnd):
    names = list(BWD_IO + BWD_DIR_IN + BWD_GRADS)
    outs = ["du", "dz", "ddelta", "dbias", "dA", "dB", "dC", "dD"]
    for m in muts:
        if m == "null":
            a[rnd.choice(names)] = None
        elif m == "null_grad":
            a[rnd.choice(["ddelta", "dA", "dB", "dC"])] = None
        elif m == "misalign":
            k = rnd.choice(names)
            if a[k] is not None:
                a[k] += rnd.choice([1, 2, 4, 8])
        elif m == "alias_out":
            o, k = rnd.choice(outs), rnd.choice(names)
            if a[k] is not None and k != o:
                a[o] = a[k] + rnd.choice([0, 4, 64])
        elif m == "ws_short":
            a["ws_bytes"] = max(0, a["ws_bytes"] - rnd.choice([1, 256, 1 << 20]))
        elif m == "ws_null":
            a["ws"] = None
        elif m == "ws_misalign":
            if a["ws"] is not None:
                a["ws"] += rnd.choice([4, 8, 12])
        elif m == "ws_over_out":
            k = rnd.choice(outs + ["u", "B"])
            if a[k] is not None:
                a["ws"] = a[k] + rnd.choice([0, 16])
        elif m == "no_z":
            a["z"] = None


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(bwd_calls())
def test_validate_bwd_matches_the_rules(lib, call):
    b, d, L, N, io, bc, muts, rnd = call
    valid = b > 0 and d > 0 and L > 0 and N == 16 and io in (0, 1) and bc in (0, 1)
    need = int(lib.sscan_bwd_workspace_bytes(b, d, L, N, 0)) if valid else 0
    a = bwd_layout(b, d, L, io if io in (0, 1) else 0, bc if bc in (0, 1) else 0, need)
    bwd_mutate(a, muts, rnd)
    g = sscan.DirGrads(a["ddelta"], a["dbias"], a["dA"], a["dB"], a["dC"], a["dD"])
    got = lib.sscan_validate_bwd(a["u"], a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"], a["z"], a["dout"],
                                 a["du"], a["dz"], ctypes.byref(g), b, d, L, N, 0, io, bc, a["ws"], a["ws_bytes"])
    want = bwd_expected(a, b, d, L, N, io, bc, need)
    if want:
        assert got in want, (got, want, muts, (b, d, L, N, io, bc))
    else:
        assert got == OK, (got, muts, (b, d, L, N, io, bc))
