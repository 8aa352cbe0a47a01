"""Python front of the fp64 selective-scan oracle (``sscan_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the HIP path never does.

``build()`` compiles the C source with gcc (-O2, no fast-math).  ``sscan_fwd`` and
``sscan_bidir`` take float64 numpy arrays in the layouts of the C file and return
the gated output in float64 (never rounded to a storage dtype).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sscan_oracle.c")
SRC_BWD = os.path.join(HERE, "sscan_oracle_bwd.c")
SRC_CONV = os.path.join(HERE, "sscan_oracle_conv.c")
LIB = os.path.join(HERE, "liboracle_sscan.so")
SOURCES = (SRC, SRC_BWD, SRC_CONV)

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into ``liboracle_sscan.so`` next to its source."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, SRC, SRC_BWD, SRC_CONV, "-lm", "-lpthread"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.environ.get("SSCAN_ORACLE_LIB") and not os.path.exists(LIB):
            build(force=True)
        # SSCAN_ORACLE_LIB: another build of the same sources (the sanitizer build of
        # the tests) to load instead
        lib = ctypes.CDLL(os.environ.get("SSCAN_ORACLE_LIB") or LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        INT = ctypes.c_int
        lib.oracle_sscan_fwd.argtypes = [P, P, P, INT, P, P, P, P, P, P, I64, I64, I64, I64, INT, P, P, INT]
        lib.oracle_sscan_fwd.restype = INT
        lib.oracle_sscan_bidir.argtypes = [P, P, P] + [P] * 12 + [INT, I64, I64, I64, I64, INT]
        lib.oracle_sscan_bidir.restype = INT
        lib.oracle_sscan_bwd.argtypes = [P, P, P, P, P, INT, P, P, P, INT, I64, I64, I64, I64, INT]
        lib.oracle_sscan_bwd.restype = INT
        lib.oracle_sscan_bwd_state.argtypes = [P, P, P, P, P, INT, P, P, P, INT, I64, I64, I64, I64, P, P, P, INT]
        lib.oracle_sscan_bwd_state.restype = INT
        lib.oracle_conv1d.argtypes = [P, P, P, P, I64, I64, I64, I64, INT, INT]
        lib.oracle_conv1d.restype = INT
        lib.oracle_softplus_f64.argtypes = [ctypes.c_double]
        lib.oracle_softplus_f64.restype = ctypes.c_double
        lib.oracle_silu_f64.argtypes = [ctypes.c_double]
        lib.oracle_silu_f64.restype = ctypes.c_double
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def sscan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, reverse=False,
              h0=None, return_last_state=False, nthreads: int = 1):
    """One direction; returns out [b, d, L] (and h_last [b, d, N] if asked)."""
    u = _c64(u)
    b, d, L = u.shape
    A = _c64(A)
    N = A.shape[1]
    delta = _c64(delta, (b, d, L))
    B = _c64(B, (b, N, L))
    C = _c64(C, (b, N, L))
    D = _c64(D, (d,))
    z = _c64(z, (b, d, L))
    bias = _c64(delta_bias, (d,))
    h0 = _c64(h0, (b, d, N))
    out = np.empty((b, d, L), dtype=np.float64)
    hl = np.empty((b, d, N), dtype=np.float64) if return_last_state else None
    st = _load().oracle_sscan_fwd(_p(u), _p(delta), _p(bias), int(bool(softplus)), _p(A), _p(B), _p(C),
                                  _p(D), _p(z), _p(out), b, d, L, N, int(bool(reverse)), _p(h0), _p(hl),
                                  int(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle_sscan_fwd failed with status {st}")
    return (out, hl) if return_last_state else out


def sscan_bidir(u, z, fwd: dict, rev: dict, softplus=True, nthreads: int = 1):
    """Both directions (separate parameter dicts with keys delta, A, B, C and
    optional D, delta_bias), summed and gated once."""
    u = _c64(u)
    b, d, L = u.shape
    z = _c64(z, (b, d, L))
    out = np.empty((b, d, L), dtype=np.float64)
    args = []
    keep = []
    for p in (fwd, rev):
        A = _c64(p["A"])
        N = A.shape[1]
        arrs = [_c64(p["delta"], (b, d, L)), _c64(p.get("delta_bias"), (d,)), A,
                _c64(p["B"], (b, N, L)), _c64(p["C"], (b, N, L)), _c64(p.get("D"), (d,))]
        keep.extend(arrs)
        args.extend(_p(a) for a in arrs)
    N = keep[2].shape[1]
    if keep[8].shape[1] != N:
        raise ValueError("both directions need the same dstate")
    st = _load().oracle_sscan_bidir(_p(u), _p(z), _p(out), *args, int(bool(softplus)), b, d, L, N, int(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle_sscan_bidir failed with status {st}")
    return out


GRAD_NAMES = ("ddelta", "ddelta_bias", "dA", "dB", "dC", "dD")


def sscan_bwd(u, z, g, dirs, softplus=True, reverse=False, nthreads: int = 1, h0=None, dh_last=None,
              return_dh0=False):
    """Gradients of sum(g * out) for one direction (``dirs`` = [params], scanned
    in reverse if ``reverse``) or two (``dirs`` = [forward, reverse]).  Each params
    dict has delta, A, B, C and optional D, delta_bias.  Returns
    {"du", "dz" (None without z), "dirs": [{ddelta, ddelta_bias, dA, dB, dC, dD}]}
    in float64; a gradient of an absent optional input is None.  One direction
    only: ``h0`` [b, d, N] is the forward's entry state, ``dh_last`` [b, d, N] the
    gradient reaching its final state, and with ``return_dh0`` the result also holds
    "dh0", the gradient of the entry state."""
    u = _c64(u)
    b, d, L = u.shape
    z = _c64(z, (b, d, L))
    g = _c64(g, (b, d, L))
    ndir = len(dirs)
    if ndir not in (1, 2):
        raise ValueError("one or two directions")
    N = np.asarray(dirs[0]["A"]).shape[1]
    keep, ins, outs, res = [], [], [], []
    for p in dirs:
        arrs = [_c64(p["delta"], (b, d, L)), _c64(p.get("delta_bias"), (d,)), _c64(p["A"], (d, N)),
                _c64(p["B"], (b, N, L)), _c64(p["C"], (b, N, L)), _c64(p.get("D"), (d,))]
        keep.extend(arrs)
        ins.extend(_p(a) for a in arrs)
        gr = {"ddelta": np.empty((b, d, L)), "ddelta_bias": np.empty(d) if p.get("delta_bias") is not None else None,
              "dA": np.empty((d, N)), "dB": np.empty((b, N, L)), "dC": np.empty((b, N, L)),
              "dD": np.empty(d) if p.get("D") is not None else None}
        res.append(gr)
        outs.extend(_p(gr[k]) for k in GRAD_NAMES)
    du = np.empty((b, d, L))
    dz = np.empty((b, d, L)) if z is not None else None
    rev = [int(bool(reverse))] if ndir == 1 else [0, 1]
    P = ctypes.c_void_p
    ins_a = (P * len(ins))(*[x.value if x is not None else None for x in ins])
    outs_a = (P * len(outs))(*[x.value if x is not None else None for x in outs])
    rev_a = (ctypes.c_int * ndir)(*rev)
    h0 = _c64(h0, (b, d, N))
    dh_last = _c64(dh_last, (b, d, N))
    dh0 = np.empty((b, d, N)) if return_dh0 else None
    st = _load().oracle_sscan_bwd_state(_p(u), _p(z), _p(g), _p(du), _p(dz), ndir, ins_a, rev_a, outs_a,
                                        int(bool(softplus)), b, d, L, N, _p(h0), _p(dh_last), _p(dh0), int(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle_sscan_bwd failed with status {st}")
    out = {"du": du, "dz": dz, "dirs": res}
    if return_dh0:
        out["dh0"] = dh0
    return out


def conv1d(x, w, bias=None, same=False, silu=False):
    """Depthwise 1-D convolution of each channel (causal, or 'same' for odd widths),
    plus bias, optionally followed by silu; x [batch, dim, len], w [dim, width]."""
    x = _c64(x)
    b, d, L = x.shape
    w = _c64(w)
    if w.shape[0] != d:
        raise ValueError("w must be [dim, width]")
    bias = _c64(bias, (d,))
    out = np.empty((b, d, L))
    st = _load().oracle_conv1d(_p(x), _p(w), _p(bias), _p(out), b, d, L, w.shape[1], int(bool(same)), int(bool(silu)))
    if st != 0:
        raise RuntimeError(f"oracle_conv1d failed with status {st}")
    return out


def conv1d_bwd(x, w, bias, same, silu, dout):
    """Gradients of sum(dout * conv1d(x, w, bias, same, silu)) with respect to x, w
    and the bias, by the chain rule through the two steps of ``conv1d``:
      pre[t] = bias + sum_j w[j] x[t - left + j]   (x = 0 outside [0, len))
      out[t] = silu(pre[t]) or pre[t],  silu'(p) = s (1 + p (1 - s)), s = 1 / (1 + e^-p)
    so with g = dout * out'(pre):  dx[s] = sum_j w[j] g[s + left - j] (t inside
    [0, len)), dw[j] = sum_{b,t} g[t] x[t - left + j], dbias = sum_{b,t} g[t].
    Returns (dx [b, d, L], dw [d, width], dbias [d]) in float64."""
    x = _c64(x)
    b, d, L = x.shape
    w = _c64(w)
    width = w.shape[1]
    pre = conv1d(x, w, bias, same=same, silu=False)
    g = _c64(dout, (b, d, L))
    if silu:
        s = 1.0 / (1.0 + np.exp(-pre))
        g = g * s * (1.0 + pre * (1.0 - s))
    left = (width - 1) // 2 if same else width - 1
    dx = np.zeros_like(x)
    dw = np.zeros((d, width))
    for j in range(width):
        # tap j joins x[t - left + j] to out[t]: pairs (t, s = t - left + j), both in range
        sh = j - left
        t0, t1 = max(0, -sh), min(L, L - sh)
        if t1 <= t0:
            continue
        dx[:, :, t0 + sh:t1 + sh] += w[None, :, j, None] * g[:, :, t0:t1]
        dw[:, j] = np.sum(g[:, :, t0:t1] * x[:, :, t0 + sh:t1 + sh], axis=(0, 2))
    return dx, dw, g.sum(axis=(0, 2))


def sscan_bwd_conv(x, conv_w, conv_bias, same, silu, z, g, dirs, softplus=True, reverse=False, nthreads: int = 1):
    """Backward of the scan with the convolution in front (sscan_fwd_conv /
    sscan_bidir_conv): the scan's gradients taken at u = conv1d(x) (``sscan_bwd``),
    then its du carried back through the convolution (``conv1d_bwd``).  Returns the
    dict of ``sscan_bwd`` without du, plus dx, dconv_w, dconv_b."""
    u = conv1d(x, conv_w, conv_bias, same=same, silu=silu)
    r = sscan_bwd(u, z, g, dirs, softplus=softplus, reverse=reverse, nthreads=nthreads)
    dx, dw, db = conv1d_bwd(x, conv_w, conv_bias, same, silu, r.pop("du"))
    r.update(dx=dx, dconv_w=dw, dconv_b=db)
    return r


def sscan_fwd_conv(x, conv_w, conv_bias, same, silu, delta, A, B, C, D=None, z=None, delta_bias=None,
                   softplus=True, reverse=False, nthreads: int = 1):
    """The scan of the convolved input: sscan_fwd(conv1d(x), ...)."""
    u = conv1d(x, conv_w, conv_bias, same, silu)
    return sscan_fwd(u, delta, A, B, C, D, z, delta_bias, softplus=softplus, reverse=reverse, nthreads=nthreads)


def sscan_step_conv(state, conv_state, x, conv_w, conv_bias, silu, delta, A, B, C, D=None, z=None, delta_bias=None,
                    softplus=True):
    """One decode token through the causal front-end convolution and the scan
    (Hand-written simplified Mamba2 page, section 5.2: the recurrent step keeps the
    state h and the last d_conv - 1 inputs of the convolution, and returns the new
    output, state and convolution state).  Steps, in the page's order:
      1. the window is the stored inputs (oldest first) followed by x_t;
      2. u_t is the causal convolution's output at the window's last position
         (``conv1d`` over the window, its last output: every tap inside it);
      3. one token of the scan from ``state`` (``sscan_fwd`` with h0, len 1);
      4. the convolution state drops its oldest input and appends x_t.
    Shapes: state [b, d, N]; conv_state [b, d, width - 1]; x, delta, z [b, d];
    B, C [b, N].  Returns (y [b, d], new state, new conv_state), all float64."""
    x = _c64(x)
    b, d = x.shape
    w = _c64(conv_w)
    width = w.shape[1]
    cs = _c64(conv_state, (b, d, width - 1))
    window = np.concatenate([cs, x[:, :, None]], axis=2)
    u = conv1d(window, w, conv_bias, same=False, silu=silu)[:, :, -1]
    col = lambda a: None if a is None else _c64(a)[:, :, None]
    y, h = sscan_fwd(u[:, :, None], col(delta), A, col(B), col(C), D, col(z), delta_bias, softplus=softplus,
                     h0=state, return_last_state=True)
    return y[:, :, 0], h, window[:, :, 1:].copy()


def softplus(x: float) -> float:
    return _load().oracle_softplus_f64(float(x))


def silu(x: float) -> float:
    return _load().oracle_silu_f64(float(x))


def run_inputs(x64: dict, softplus=True, nthreads: int = 1, reverse=False, gate=True):
    """Oracle on a dict from ``inputs.as_f64_dict`` (one or two directions)."""
    z = x64["z"] if gate else None
    dirs = x64["dirs"]
    if len(dirs) == 1:
        p = dirs[0]
        return sscan_fwd(x64["u"], x64["delta"], p["A"], p["B"], p["C"], p["D"], z, p["delta_bias"],
                         softplus=softplus, reverse=reverse, nthreads=nthreads)
    f, r = dirs
    return sscan_bidir(x64["u"], z, dict(f, delta=x64["delta"]), dict(r, delta=x64["delta"]),
                       softplus=softplus, nthreads=nthreads)
