"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call.

Pointers passed here are fake, never dereferenced: validation only looks at
NULL-ness, alignment, overlap and sizes.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_sscan_amd import sscan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sscan.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP, EALIAS = 0, -1, -2, -3, -4, -5, -6, -7
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    # SSCAN_TEST_LIBRARY: another build of the same library to run these checks on
    # (the sanitizer build of test_asan_host.py)
    other = os.environ.get("SSCAN_TEST_LIBRARY")
    if other:
        return sscan.load_library(other)
    if not os.path.exists(sscan.LIB_PATH):
        from selective_state_space_sscan_amd import build
        build.build()
    return sscan.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SSCAN_API\s+[\w\s\*]*?\b(sscan_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert {"sscan_fwd", "sscan_bidir", "sscan_workspace_bytes", "sscan_strerror"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_strerror_and_version(lib):
    for st in (OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP, EALIAS, 123):
        assert isinstance(sscan.strerror(st), str) and sscan.strerror(st)
    assert sscan.strerror(123) == "unknown status"
    assert lib.sscan_version() >= 100


class Fake:
    """Disjoint fake device addresses, 256-byte aligned."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes):
        p = self.next
        self.next += (nbytes + 4096) // 256 * 256 + 256
        return p


def fwd_args(b, d, L, io=0, bc=0, **over):
    f = Fake()
    ie = 2 if io == 1 else 4
    be = 2 if bc == 1 else 4
    a = dict(u=f(b * d * L * ie), delta=f(b * d * L * ie), bias=f(d * 4), softplus=1, A=f(d * 64), B=f(b * 16 * L * be),
             C=f(b * 16 * L * be), D=f(d * 4), z=f(b * d * L * ie), y=f(b * d * L * ie), b=b, d=d, L=L, N=16,
             reverse=0, io=io, bc=bc, ws=f(1 << 33), ws_bytes=1 << 33)
    a.update(over)
    return a


def call_validate_fwd(lib, a):
    return lib.sscan_validate_fwd(a["u"], a["delta"], a["bias"], a["softplus"], a["A"], a["B"], a["C"], a["D"],
                                  a["z"], a["y"], a["b"], a["d"], a["L"], a["N"], a["reverse"], a["io"], a["bc"],
                                  a["ws"], a["ws_bytes"])


def test_validate_fwd_accepts_good_arguments(lib):
    for io, bc in ((0, 0), (1, 1), (1, 0)):
        assert call_validate_fwd(lib, fwd_args(2, 64, 32, io, bc)) == OK
        assert call_validate_fwd(lib, fwd_args(1, 1536, 262144, io, bc)) == OK
    assert call_validate_fwd(lib, fwd_args(2, 64, 32, D=None, bias=None, z=None)) == OK


@pytest.mark.parametrize("name", ["u", "delta", "A", "B", "C", "y"])
def test_validate_fwd_null_required(lib, name):
    assert call_validate_fwd(lib, fwd_args(2, 64, 32, **{name: None})) == ENULL


@pytest.mark.parametrize("over,status", [
    (dict(b=-1), ESHAPE), (dict(d=-5), ESHAPE), (dict(L=-1), ESHAPE),
    (dict(b=1 << 40, d=1 << 20, L=1 << 20), ESHAPE),
    (dict(b=1 << 20, d=1, L=(1 << 16) + 1), ESHAPE),  # batch * len above 2^36
    (dict(N=8), EUNSUP), (dict(N=32), EUNSUP), (dict(io=2), EUNSUP), (dict(bc=-1), EUNSUP),
])
def test_validate_fwd_bad_sizes_and_codes(lib, over, status):
    assert call_validate_fwd(lib, dict(fwd_args(2, 64, 32), **over)) == status


def test_validate_fwd_alignment(lib):
    a = fwd_args(2, 64, 32)
    assert call_validate_fwd(lib, dict(a, u=a["u"] + 2)) == EALIGN
    assert call_validate_fwd(lib, dict(a, A=a["A"] + 1)) == EALIGN
    assert call_validate_fwd(lib, dict(a, B=a["B"] + 2)) == EALIGN
    bf = fwd_args(2, 64, 32, io=1, bc=1)
    assert call_validate_fwd(lib, dict(bf, u=bf["u"] + 2, y=bf["y"] + 2)) == OK  # bf16: 2-byte alignment suffices
    assert call_validate_fwd(lib, dict(bf, y=bf["y"] + 1)) == EALIGN


def test_validate_fwd_aliasing(lib):
    a = fwd_args(2, 64, 32)
    assert call_validate_fwd(lib, dict(a, y=a["u"])) == EALIAS
    assert call_validate_fwd(lib, dict(a, y=a["z"] + 64)) == EALIAS
    assert call_validate_fwd(lib, dict(a, y=a["B"])) == EALIAS


def test_grids_stay_under_2_32_work_items(lib):
    """A dispatch covers fewer than 2^32 work-items per grid dimension: a call whose
    kernels would need more is refused before any launch (SSCAN_ERR_SHAPE), a call
    just inside is accepted.  B/C staging runs 256 threads per 64 tokens of each
    batch row: batch 2^26 x len 1 needs 2^34; batch 2^23 needs 2^31."""
    for batch, expect in ((1 << 26, ESHAPE), (1 << 23, OK)):
        a = fwd_args(batch, 64, 1, io=1, bc=1)
        assert call_validate_fwd(lib, dict(a, ws=1 << 60, ws_bytes=1 << 62)) == expect, batch
    # the same bound through batch x len: 2^16 rows of 2^16 tokens
    assert call_validate_fwd(lib, dict(fwd_args(1 << 16, 64, 1 << 16), ws=1 << 60, ws_bytes=1 << 62)) == ESHAPE


def test_empty_call_is_ok_even_without_pointers(lib):
    a = fwd_args(0, 64, 32, u=None, y=None, delta=None)
    assert call_validate_fwd(lib, a) == OK
    assert call_validate_fwd(lib, fwd_args(2, 64, 0)) == OK


def staging_bytes(ndir, b, L):
    # B and C re-laid token-major in fp32: 32 floats per token and direction
    return (ndir * b * L * 32 + 63) // 64 * 64 * 4


def park_bytes(b, d, L):
    # bidirectional meeting buffers of an unsplit sequence longer than 64 tokens,
    # kept in global memory: per (batch row, 64-channel group) L tokens x 64 lanes
    return (b * ((d + 63) // 64) * L * 64 + 63) // 64 * 64 * 4


def test_workspace_rules(lib):
    # unsplit sequence: B/C staging, plus global meeting buffers for a bidirectional
    # one longer than 64 tokens
    assert lib.sscan_workspace_bytes(128, 768, 64, 16, 1) == staging_bytes(2, 128, 64)
    short = lib.sscan_workspace_bytes(128, 768, 197, 16, 1)
    assert short == staging_bytes(2, 128, 197) + park_bytes(128, 768, 197)
    assert lib.sscan_workspace_bytes(128, 768, 197, 16, 0) == staging_bytes(1, 128, 197)
    assert lib.sscan_workspace_bytes(64, 384, 197, 16, 1) == staging_bytes(2, 64, 197) + park_bytes(64, 384, 197)
    assert lib.sscan_workspace_bytes(2, 64, 32, 16, 0) == staging_bytes(1, 2, 32)
    assert call_validate_fwd(lib, fwd_args(2, 64, 32, ws=None, ws_bytes=0)) == EWS
    long_f = lib.sscan_workspace_bytes(1, 1536, 262144, 16, 0)
    long_b = lib.sscan_workspace_bytes(8, 192, 16384, 16, 1)
    assert long_f > 0 and long_b > 0
    # staging plus per-segment aggregates: a few percent of the inputs at most
    assert staging_bytes(1, 1, 262144) < long_f < 0.05 * (1536 * 262144 * 2 * 4)
    assert call_validate_fwd(lib, fwd_args(1, 1536, 262144, ws=None, ws_bytes=0)) == EWS
    assert call_validate_fwd(lib, fwd_args(1, 1536, 262144, ws_bytes=long_f - 1)) == EWS
    a = fwd_args(1, 1536, 262144, ws_bytes=long_f)
    assert call_validate_fwd(lib, a) == OK
    assert call_validate_fwd(lib, dict(a, ws=a["ws"] + 4)) == EALIGN
    assert lib.sscan_workspace_bytes(1, 1536, 262144, 8, 0) == 0  # unsupported dstate: reported by the call


def test_validate_bidir(lib):
    f = Fake()
    b, d, L = 8, 192, 16384
    n_io, n_bc = b * d * L * 2, b * 16 * L * 2
    u, z, y, delta = f(n_io), f(n_io), f(n_io), f(n_io)
    mk = lambda: sscan.DirParams(delta, f(d * 4), f(d * 64), f(n_bc), f(n_bc), f(d * 4))
    pf, pr = mk(), mk()
    ws = lib.sscan_workspace_bytes(b, d, L, 16, 1)
    wsp = f(ws)
    V = lambda *a: lib.sscan_validate_bidir(*a)
    assert V(u, z, y, ctypes.byref(pf), ctypes.byref(pr), 1, b, d, L, 16, 1, 1, wsp, ws) == OK
    assert V(u, z, y, None, ctypes.byref(pr), 1, b, d, L, 16, 1, 1, wsp, ws) == ENULL
    bad = sscan.DirParams(delta, None, None, pf.B, pf.C, None)
    assert V(u, z, y, ctypes.byref(pf), ctypes.byref(bad), 1, b, d, L, 16, 1, 1, wsp, ws) == ENULL
    assert V(u, z, y, ctypes.byref(pf), ctypes.byref(pr), 1, b, d, L, 16, 1, 1, None, 0) == EWS
    assert V(u, z, pf.B, ctypes.byref(pf), ctypes.byref(pr), 1, b, d, L, 16, 1, 1, wsp, ws) == EALIAS
    assert V(u, z, y, ctypes.byref(pf), ctypes.byref(pr), 1, b, d, L, 16, 1, 1, y + 128, ws) == EALIAS


def test_run_entry_points_reject_before_any_hip_call(lib):
    """The run entry points return validation errors without touching HIP (no GPU here)."""
    a = fwd_args(2, 64, 32, u=None)
    st = lib.sscan_fwd(a["u"], a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"], a["z"], a["y"],
                       2, 64, 32, 16, 0, None, 0, 0, None, 0)
    assert st == ENULL
    st = lib.sscan_fwd(1 << 40, a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"], a["z"], a["y"],
                       2, 64, 32, 12, 0, None, 0, 0, None, 0)
    assert st == EUNSUP
    st = lib.sscan_bidir(None, None, None, None, None, 1, 2, 64, 32, 16, None, 0, 0, None, 0)
    assert st == ENULL


def test_noalloc_rejects_before_any_hip_call(lib):
    """sscan_fwd_noalloc refuses a call that needs more workspace than its scratch
    array, and every invalid argument, without touching HIP (no GPU here)."""
    ETOO = -8
    assert sscan.strerror(ETOO) != "unknown status"
    b, d, L = 1, 1536, 262144
    assert sscan.workspace_bytes(b, d, L) > sscan.NOALLOC_SCRATCH_BYTES
    a = fwd_args(b, d, L, io=1)
    call = lambda a, N=16: lib.sscan_fwd_noalloc(a["u"], a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"],
                                                 a["z"], a["y"], a["b"], a["d"], a["L"], N, 0, None, a["io"], a["bc"])
    assert call(a) == ETOO
    small = fwd_args(2, 64, 300, io=1)
    assert call(dict(small, u=None)) == ENULL
    assert call(dict(small, y=small["u"])) == EALIAS
    assert call(small, N=8) == EUNSUP
    assert call(dict(small, b=-1)) == ESHAPE


# --- state I/O and single-step decode ------------------------------------------------------------

def call_validate_state(lib, a, h0, hl):
    return lib.sscan_validate_fwd_state(a["u"], a["delta"], a["bias"], a["softplus"], a["A"], a["B"], a["C"], a["D"],
                                        a["z"], a["y"], h0, hl, a["b"], a["d"], a["L"], a["N"], a["reverse"], a["io"],
                                        a["bc"], a["ws"], a["ws_bytes"])


def test_validate_fwd_state(lib):
    f = Fake()
    f.next = 1 << 46  # clear of the addresses fwd_args hands out
    a = fwd_args(2, 64, 300, io=1)
    sb = 2 * 64 * 16 * 4
    h0, hl = f(sb), f(sb)
    assert call_validate_state(lib, a, h0, hl) == OK
    assert call_validate_state(lib, a, None, hl) == OK
    assert call_validate_state(lib, a, h0, None) == OK
    assert call_validate_state(lib, a, h0, h0) == OK            # the state updated in place
    assert call_validate_state(lib, a, h0, h0 + 64) == EALIAS   # partial overlap
    assert call_validate_state(lib, a, h0, h0 + 4) == EALIGN    # state buffers need 16 bytes
    assert call_validate_state(lib, a, h0, a["u"]) == EALIAS
    assert call_validate_state(lib, a, h0, a["A"]) == EALIAS
    assert call_validate_state(lib, a, h0, a["ws"] + 256) == EALIAS
    assert call_validate_state(lib, dict(a, y=h0), h0, hl) == EALIAS
    assert call_validate_state(lib, dict(a, u=None), h0, hl) == ENULL
    # an empty sequence with a final state is a valid call (the state passes through)
    assert call_validate_state(lib, fwd_args(2, 64, 0), h0, hl) == OK


def step_args(b, d, io=0, bc=0, **over):
    f = Fake()
    ie = 2 if io == 1 else 4
    be = 2 if bc == 1 else 4
    a = dict(state=f(b * d * 64), u=f(b * d * ie), delta=f(b * d * ie), bias=f(d * 4), softplus=1, A=f(d * 64),
             B=f(b * 16 * be), C=f(b * 16 * be), D=f(d * 4), z=f(b * d * ie), y=f(b * d * ie), b=b, d=d, N=16,
             io=io, bc=bc)
    a.update(over)
    return a


def call_validate_step(lib, a):
    return lib.sscan_validate_step(a["state"], a["u"], a["delta"], a["bias"], a["softplus"], a["A"], a["B"], a["C"],
                                   a["D"], a["z"], a["y"], a["b"], a["d"], a["N"], a["io"], a["bc"])


def test_validate_step(lib):
    for io, bc in ((0, 0), (1, 1), (1, 0)):
        assert call_validate_step(lib, step_args(4, 1536, io, bc)) == OK
    assert call_validate_step(lib, step_args(4, 100, D=None, bias=None, z=None)) == OK
    for name in ("state", "u", "delta", "A", "B", "C", "y"):
        assert call_validate_step(lib, step_args(4, 100, **{name: None})) == ENULL, name
    a = step_args(4, 100)
    assert call_validate_step(lib, dict(a, N=8)) == EUNSUP
    assert call_validate_step(lib, dict(a, b=-1)) == ESHAPE
    assert call_validate_step(lib, dict(a, state=a["state"] + 4)) == EALIGN
    assert call_validate_step(lib, dict(a, A=a["A"] + 4)) == EALIGN
    assert call_validate_step(lib, dict(a, B=a["B"] + 8)) == EALIGN
    ab = step_args(4, 100, io=1, bc=1)
    assert call_validate_step(lib, dict(ab, B=ab["B"] + 8, C=ab["C"] + 8)) == OK  # bf16: 8 bytes suffice
    assert call_validate_step(lib, dict(ab, C=ab["C"] + 4)) == EALIGN
    assert call_validate_step(lib, dict(a, y=a["state"])) == EALIAS
    assert call_validate_step(lib, dict(a, y=a["u"])) == EALIAS
    assert call_validate_step(lib, dict(a, state=a["B"])) == EALIAS
    assert call_validate_step(lib, step_args(0, 100, state=None, u=None)) == OK  # empty
    st = lib.sscan_step(None, a["u"], a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"], a["z"], a["y"],
                        4, 100, 16, None, 0, 0)
    assert st == ENULL


def test_validate_step_conv(lib):
    """The decode step through the causal convolution: the step's checks, a causal
    convolution of 1..4 taps, and a window buffer that overlaps nothing else."""
    f = Fake()
    f.next = 1 << 47

    def call(a, cs, width=4, same=0, silu=1, weight=True, bias=True):
        w = f(a["d"] * width * 4) if weight else None
        cb = f(a["d"] * 4) if bias else None
        cp = sscan.ConvParams(w, cb, width, same, silu)
        return lib.sscan_validate_step_conv(a["state"], cs, a["u"], ctypes.byref(cp), a["delta"], a["bias"], 1, a["A"],
                                            a["B"], a["C"], a["D"], a["z"], a["y"], a["b"], a["d"], a["N"], a["io"],
                                            a["bc"])

    for io in (0, 1):
        a = step_args(4, 100, io, io)
        cs = f(4 * 100 * 3 * 4)
        assert call(a, cs) == OK
        assert call(a, None, width=1) == OK      # no window to keep
        assert call(a, None) == ENULL
        assert call(a, cs, same=1, width=3) == EUNSUP
        assert call(a, cs, width=5) == EUNSUP
        assert call(a, cs, weight=False) == ENULL
        assert call(a, cs + (1 if io else 2)) == EALIGN
        assert call(a, a["u"]) == EALIAS          # the window overlaps x
        assert call(a, a["state"] + 64) == EALIAS
        assert call(dict(a, y=None), cs) == ENULL
    assert call(step_args(0, 100), None) == OK  # empty
    a = step_args(4, 100)
    cp = sscan.ConvParams(None, None, 4, 0, 0)
    st = lib.sscan_step_conv(a["state"], None, a["u"], ctypes.byref(cp), a["delta"], a["bias"], 1, a["A"], a["B"],
                             a["C"], a["D"], a["z"], a["y"], 4, 100, 16, None, 0, 0)
    assert st == ENULL  # rejected before any HIP call


def test_validate_bwd_state(lib):
    """The state backward: the backward's checks plus h0, dh_last (inputs) and dh0
    (output), 16-byte aligned [batch, dim, 16] float32."""
    f = Fake()
    f.next = 1 << 44
    b, d, L = 2, 64, 300
    a = fwd_args(b, d, L)
    dout, du, dz = f(b * d * L * 4), f(b * d * L * 4), f(b * d * L * 4)
    gs = sscan.DirGrads(f(b * d * L * 4), f(d * 4), f(d * 64), f(b * 16 * L * 4), f(b * 16 * L * 4), f(d * 4))
    h0, dhl, dh0 = f(b * d * 64), f(b * d * 64), f(b * d * 64)
    ws = lib.sscan_bwd_workspace_bytes(b, d, L, 16, 0)
    wsp = f(ws)

    def call(h0=h0, dhl=dhl, dh0=dh0):
        return lib.sscan_validate_bwd_state(a["u"], a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"], a["z"],
                                            dout, h0, dhl, du, dz, ctypes.byref(gs), dh0, b, d, L, 16, 0, 0, 0, wsp,
                                            ws)

    assert call() == OK
    assert call(h0=None, dhl=None, dh0=None) == OK
    assert call(h0=h0 + 4) == EALIGN
    assert call(dh0=dh0 + 8) == EALIGN
    assert call(dh0=du) == EALIAS            # dh0 over an output
    assert call(dh0=h0) == EALIAS            # ... or over the entry state
    assert call(h0=gs.dB) == EALIAS          # an input under an output
    assert call(dhl=wsp) == EALIAS
    assert lib.sscan_validate_bwd_state(a["u"], a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"], a["z"], dout,
                                        h0, dhl, du, dz, None, dh0, b, d, L, 16, 0, 0, 0, wsp, ws) == ENULL


def test_validate_bwd_conv(lib):
    """The backward through the convolution: the scan backward's checks with x and
    dx in u's and du's places, the convolution's, its weight and bias gradients, and
    the larger workspace."""
    f = Fake()
    f.next = 1 << 45
    b, d, L = 2, 64, 300
    ws_need = lib.sscan_bwd_conv_workspace_bytes(b, d, L, 16, 0, 0)
    assert ws_need > lib.sscan_bwd_workspace_bytes(b, d, L, 16, 0)
    a = fwd_args(b, d, L)
    dout, dx, dz = f(b * d * L * 4), f(b * d * L * 4), f(b * d * L * 4)
    gr = [f(b * d * L * 4), f(d * 4), f(d * 64), f(b * 16 * L * 4), f(b * 16 * L * 4), f(d * 4)]
    gs = sscan.DirGrads(*gr)
    wsp = f(ws_need)

    def call(w=True, bias=True, width=4, same=0, dw="ok", db="ok", ws=wsp, ws_bytes=ws_need, xx=None):
        cw = f(d * width * 4) if w else None
        cb = f(d * 4) if bias else None
        cp = sscan.ConvParams(cw, cb, width, same, 1)
        dwp = f(d * width * 4) if dw == "ok" else dw
        dbp = f(d * 4) if db == "ok" else db
        return lib.sscan_validate_bwd_conv(a["u"] if xx is None else xx, ctypes.byref(cp), a["delta"], a["bias"], 1,
                                           a["A"], a["B"], a["C"], a["D"], a["z"], dout, dx, dz, ctypes.byref(gs),
                                           dwp, dbp, b, d, L, 16, 0, 0, 0, ws, ws_bytes)

    assert call() == OK
    assert call(bias=False, db=None) == OK       # no bias: no bias gradient
    assert call(db=None) == ENULL                # a bias needs its gradient
    assert call(dw=None) == ENULL
    assert call(w=False) == ENULL
    assert call(width=4, same=1) == EUNSUP
    assert call(ws_bytes=ws_need - 256) == EWS
    assert call(ws=None, ws_bytes=0) == EWS
    assert call(dw=dx) == EALIAS                 # a conv gradient overlapping dx
    assert call(dw=wsp + 1024 * 1024) == EALIAS  # ... or the workspace's back part
    assert call(db=a["u"]) == EALIAS
    assert call(xx=None) == OK


# --- backward -------------------------------------------------------------------------------

def bwd_call(lib, a, g, dout, du, dz):
    gs = sscan.DirGrads(*g)
    return lib.sscan_validate_bwd(a["u"], a["delta"], a["bias"], 1, a["A"], a["B"], a["C"], a["D"], a["z"], dout,
                                  du, dz, ctypes.byref(gs), a["b"], a["d"], a["L"], 16, 0, a["io"], a["bc"], a["ws"],
                                  a["ws_bytes"])


def test_validate_bwd(lib):
    f = Fake()
    f.next = 1 << 46
    b, d, L = 2, 64, 300
    a = fwd_args(b, d, L)
    io, bc = b * d * L * 4, b * 16 * L * 4
    dout, du, dz = f(io), f(io), f(io)
    g = [f(io), f(d * 4), f(d * 64), f(bc), f(bc), f(d * 4)]
    ws = lib.sscan_bwd_workspace_bytes(b, d, L, 16, 0)
    assert ws > lib.sscan_workspace_bytes(b, d, L, 16, 0)
    a = dict(a, ws=f(ws), ws_bytes=ws)
    assert bwd_call(lib, a, g, dout, du, dz) == OK
    assert bwd_call(lib, a, g, dout, du, None) == ENULL            # z given: dz required
    assert bwd_call(lib, dict(a, z=None), g, dout, du, None) == OK
    assert bwd_call(lib, a, g, None, du, dz) == ENULL
    assert bwd_call(lib, a, [None] + g[1:], dout, du, dz) == ENULL  # ddelta
    assert bwd_call(lib, a, g[:2] + [None] + g[3:], dout, du, dz) == ENULL  # dA
    assert bwd_call(lib, a, g[:1] + [None] + g[2:5] + [None], dout, du, dz) == OK  # optional grads
    assert bwd_call(lib, a, g, dout, a["u"], dz) == EALIAS          # output over an input
    assert bwd_call(lib, a, g, dout, du, du) == EALIAS              # two outputs
    assert bwd_call(lib, a, g[:3] + [a["ws"] + 256] + g[4:], dout, du, dz) == EALIAS  # over the workspace
    assert bwd_call(lib, dict(a, ws_bytes=ws - 1), g, dout, du, dz) == EWS
    assert bwd_call(lib, a, g, dout + 2, du, dz) == EALIGN
    # empty sequence: only the gradients with elements are needed
    e = fwd_args(b, d, 0, u=None, delta=None, y=None)
    assert bwd_call(lib, dict(e, ws=None, ws_bytes=0), [None, g[1], g[2], None, None, g[5]], None, None, None) == OK
    assert bwd_call(lib, dict(e, ws=None, ws_bytes=0), [None, g[1], None, None, None, g[5]], None, None, None) == ENULL


# --- front-end convolution --------------------------------------------------------------------

def test_validate_conv1d(lib):
    f = Fake()
    f.next = 1 << 46
    b, d, L = 2, 64, 100
    x, y, w, bias = f(b * d * L * 4), f(b * d * L * 4), f(d * 16), f(d * 4)
    V = lambda cp, **kw: lib.sscan_validate_conv1d(kw.get("x", x), ctypes.byref(cp) if cp else None, kw.get("y", y),
                                                   b, d, L, kw.get("io", 0))
    C = lambda width, same=0, silu=0, weight=w, bias_=bias: sscan.ConvParams(weight, bias_, width, same, silu)
    for width in (1, 2, 3, 4):
        assert V(C(width)) == OK
    assert V(C(3, same=1)) == OK and V(C(1, same=1)) == OK and V(C(4, silu=1)) == OK
    assert V(C(5)) == EUNSUP and V(C(0)) == EUNSUP
    assert V(C(2, same=1)) == EUNSUP and V(C(5, same=1)) == EUNSUP  # centred needs an odd width <= 3
    assert V(C(3, silu=2)) == EUNSUP
    assert V(C(3, weight=None)) == ENULL and V(None) == ENULL
    assert V(C(3), y=x) == EALIAS and V(C(3), y=w) == EALIAS
    assert V(C(3, weight=w + 2)) == EALIGN
    assert V(C(3), y=y + 2, io=1) == OK and V(C(3), y=y + 1, io=1) == EALIGN


# --- 2-D visiting orders -------------------------------------------------------------------------

@pytest.mark.parametrize("h,w", [(1, 1), (1, 7), (6, 1), (2, 2), (5, 5), (4, 6), (7, 3), (16, 16), (13, 9)])
def test_spiral_order_matches_the_oracle(lib, h, w):
    """The library's spiral (host code) and the oracle's, written separately from
    the same description, agree index for index."""
    from oracle import orders

    assert sscan.spiral_order(h, w).tolist() == orders.spiral_order(h, w).tolist()


def test_spiral_order_rejects_bad_sizes(lib):
    assert lib.sscan_spiral_order(-1, 3, None) == ESHAPE
    assert lib.sscan_spiral_order(3, 3, None) == ENULL
    assert lib.sscan_spiral_order(0, 3, None) == OK


def test_validate_multi(lib):
    f = Fake()
    f.next = 1 << 46
    b, d, h, w = 2, 64, 8, 12
    L = h * w
    io, bc = b * d * L * 4, b * 16 * L * 4
    u, z, y, index = f(io), f(io), f(io), f(L * 4)
    mk = lambda: sscan.DirParams(f(io), f(d * 4), f(d * 64), f(bc), f(bc), f(d * 4))
    dirs = (sscan.DirParams * 4)(*[mk() for _ in range(4)])
    K = lambda *k: (ctypes.c_int * len(k))(*k)
    kinds = K(0, 1, 2, 3)
    ws = lib.sscan_multi_workspace_bytes(b, d, h, w, 16, kinds, 4, 0, 0)
    assert ws > 0
    wsp = f(ws)
    V = lambda kk, n, **kw: lib.sscan_validate_multi(kw.get("u", u), z, kw.get("y", y), dirs, kk, n,
                                                     kw.get("index", None), 1, b, d, kw.get("h", h), w, 16, 0, 0,
                                                     kw.get("ws", wsp), kw.get("ws_bytes", ws))
    assert V(kinds, 4) == OK
    assert V(K(0, 0), 2) == EUNSUP          # a kind twice
    assert V(K(6), 1) == EUNSUP             # unknown kind
    assert V(kinds, 0) == EUNSUP and V(kinds, 7) == EUNSUP
    assert V(K(4), 1) == ENULL              # the index orders need the index
    ws4 = lib.sscan_multi_workspace_bytes(b, d, h, w, 16, K(4), 1, 0, 0)
    assert V(K(4), 1, index=index, ws_bytes=ws4) == OK
    assert V(kinds, 4, ws_bytes=ws - 1) == EWS
    assert V(kinds, 4, ws=wsp + 16) == EALIGN  # 256-byte aligned workspace
    assert V(kinds, 4, y=u) == EALIAS
    assert V(kinds, 4, h=-1) == ESHAPE


def test_validate_multi_bwd(lib):
    f = Fake()
    f.next = 1 << 46
    b, d, h, w = 2, 64, 8, 12
    L = h * w
    io, bc = b * d * L * 4, b * 16 * L * 4
    u, z, dout, du, dz, index = f(io), f(io), f(io), f(io), f(io), f(L * 4)
    mk = lambda: sscan.DirParams(f(io), f(d * 4), f(d * 64), f(bc), f(bc), f(d * 4))
    mg = lambda: [f(io), f(d * 4), f(d * 64), f(bc), f(bc), f(d * 4)]
    dirs = (sscan.DirParams * 4)(*[mk() for _ in range(4)])
    grads = [mg() for _ in range(4)]
    G = lambda gs: (sscan.DirGrads * len(gs))(*[sscan.DirGrads(*g) for g in gs])
    K = lambda *k: (ctypes.c_int * len(k))(*k)
    kinds = K(0, 1, 2, 3)
    ws = lib.sscan_multi_bwd_workspace_bytes(b, d, h, w, 16, kinds, 4, 0, 0)
    assert ws > lib.sscan_multi_workspace_bytes(b, d, h, w, 16, kinds, 4, 0, 0)
    wsp = f(ws)

    def V(kk, n, gs=grads, **kw):
        return lib.sscan_validate_multi_bwd(kw.get("u", u), kw.get("z", z), kw.get("dout", dout), kw.get("du", du),
                                            kw.get("dz", dz), dirs, G(gs), kk, n, kw.get("index", None), 1,
                                            kw.get("b", b), d, kw.get("h", h), w, 16, 0, 0, kw.get("ws", wsp),
                                            kw.get("ws_bytes", ws))

    assert V(kinds, 4) == OK
    assert V(kinds, 4, z=None, dz=None) == OK
    assert V(kinds, 4, dz=None) == ENULL                           # z given: dz required
    assert V(kinds, 4, dout=None) == ENULL
    assert V(K(4), 1) == ENULL                                     # the index orders need the index
    ws4 = lib.sscan_multi_bwd_workspace_bytes(b, d, h, w, 16, K(4), 1, 0, 0)
    assert V(K(4), 1, index=index, ws_bytes=ws4) == OK
    assert V(K(4), 1, index=index, du=index, ws_bytes=ws4) == EALIAS  # an output over the index
    assert V(K(0, 0), 2) == EUNSUP
    bad = [list(g) for g in grads]
    bad[2][0] = None                                               # a direction's ddelta
    assert V(kinds, 4, bad) == ENULL
    bad = [list(g) for g in grads]
    bad[3][4] = grads[1][4]                                        # two directions' dC in one buffer
    assert V(kinds, 4, bad) == EALIAS
    bad = [list(g) for g in grads]
    bad[1][3] = dirs[0].B                                          # a gradient over an input
    assert V(kinds, 4, bad) == EALIAS
    assert V(kinds, 4, du=dz) == EALIAS
    assert V(kinds, 4, ws_bytes=ws - 1) == EWS
    assert V(kinds, 4, ws=wsp + 16) == EALIGN
    assert V(kinds, 4, dout=dout + 2) == EALIGN
    assert V(kinds, 4, h=-1) == ESHAPE
    # an empty map: only the parameter gradients with elements are needed
    assert V(kinds, 4, [[None, g[1], g[2], None, None, g[5]] for g in grads], h=0, u=None, z=None, dout=None,
             du=None, dz=None, ws=None, ws_bytes=0) == OK
    assert lib.sscan_multi_bwd_workspace_bytes(b, d, 0, w, 16, kinds, 4, 0, 0) == 0


def test_bwd_plan_splits():
    """How backward calls are split: a window's channel groups go to about 32768
    blocks per launch (one direction per launch) with at least 16 groups per block,
    the last block taking what remains."""
    plan = sscan.bwd_plan
    assert plan(1, 1536, 262144) == dict(nwin=8192, csplit=4, gps=96, run_len=24, nrun=342)
    assert plan(8, 192, 16384, bidir=True) == dict(nwin=512, csplit=3, gps=16, run_len=3, nrun=171)
    # a short sequence whose whole-sequence runs still give 3,072 chain waves is one run
    assert plan(128, 768, 197, bidir=True) == dict(nwin=7, csplit=12, gps=16, run_len=7, nrun=1)
    assert plan(64, 384, 197, bidir=True)["run_len"] == 1
    p = plan(64, 384, 197, bidir=True)
    assert (p["csplit"], p["gps"]) == (6, 16)
    # fewer than 32 groups: one block per window
    assert plan(2, 64, 300)["csplit"] == 1 and plan(2, 124, 300)["csplit"] == 1
    # 51 groups: three blocks of 17, the last group partial
    p = plan(2, 202, 150, bidir=True)
    assert (p["csplit"], p["gps"]) == (3, 17)
    # 33 groups: two blocks, 17 + 16
    p = plan(1, 130, 777)
    assert (p["csplit"], p["gps"]) == (2, 17)
    for b, d, L in [(1, 1536, 262144), (3, 1000, 5000), (2, 202, 150), (1, 4, 1)]:
        p = plan(b, d, L)
        groups = -(-d // 4)
        assert p["nwin"] == -(-L // 32) and p["csplit"] * p["gps"] >= groups > (p["csplit"] - 1) * p["gps"]
        assert p["nrun"] * p["run_len"] >= p["nwin"] > (p["nrun"] - 1) * p["run_len"]
    with pytest.raises(sscan.SScanError):
        plan(1, 64, 100, dstate=8)


def test_scan_plan_splits():
    """How calls are split: short sequences whole; long one-direction sequences in
    512-token segments (1536 channels), one per aggregate run; long bidirectional ones in 64-token
    segments, grouped in aggregate runs only when one wave per segment would exceed
    four rounds of resident waves."""
    plan = sscan.scan_plan
    assert plan(128, 768, 197, bidir=True) == dict(seg_len=197, nseg=1, run_len=1, nrun=1)
    assert plan(2, 64, 256) == dict(seg_len=256, nseg=1, run_len=1, nrun=1)
    assert plan(1, 1536, 262144) == dict(seg_len=512, nseg=512, run_len=1, nrun=512)
    assert plan(8, 192, 16384, bidir=True) == dict(seg_len=64, nseg=256, run_len=1, nrun=256)
    long_b = plan(1, 64, 1 << 20, bidir=True)
    assert long_b["seg_len"] == 64 and long_b["run_len"] == 2 and long_b["nrun"] * 2 == long_b["nseg"]
    assert plan(1, 192, 512 * 512, bidir=True)["run_len"] == 2
    assert plan(1, 1536, 512 * 512, bidir=True)["run_len"] == 16
    with pytest.raises(sscan.SScanError):
        plan(1, 64, 100, dstate=8)
