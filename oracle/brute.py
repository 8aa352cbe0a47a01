"""Materialised O(L^2) form of the selective scan, used to certify the oracle.

TEST INFRASTRUCTURE ONLY.  This is deliberately a different computation from the
sequential recurrence in ``sscan_oracle.c``: the recurrence is unrolled into the
"matrix" (dual) form that the Hand-written simplified Mamba2 page describes in
section 3.1 (all past inputs weighted by a decay matrix and summed at once), and
that, with input-independent parameters, reduces to the convolution kernel
K = (CB, CAB, CA^2B, ...) of section 2.3 of the same page.

Forward direction, token t:
    y_t = sum_{s<=t} [ sum_n C[n,t] * exp(A[n] * sum_{r=s+1..t} dt_r) * dt_s * B[n,s] ] * u_s
          + D * u_t
Reverse direction (scan with t descending), token t:
    y_t = sum_{s>=t} [ sum_n C[n,t] * exp(A[n] * sum_{r=t..s-1} dt_r) * dt_s * B[n,s] ] * u_s
          + D * u_t
with dt = softplus(delta + bias) (numpy's logaddexp(0, x)) or delta + bias.
Bidirectional output = (y_forward + y_reverse) * silu(z).

``brute_mp`` evaluates the same sums with mpmath at a chosen precision, for tiny
inputs only.
"""
from __future__ import annotations

import numpy as np


def _dt_numpy(delta, bias, softplus):
    x = delta + (0.0 if bias is None else bias[None, :, None])
    return np.logaddexp(0.0, x) if softplus else x


def brute_dir(u, delta, A, B, C, D=None, delta_bias=None, softplus=True, reverse=False, h0=None):
    """Ungated output of one direction (float64 numpy), O(b*d*L^2*N).

    With an entry state h0 [b, d, N] (the state before the first scanned token),
    every output also reads that state decayed over all tokens scanned so far:
    y_t += sum_n C[n,t] exp(A_n E_t) h0_n, E_t = sum_{r<=t} dt_r forward,
    sum_{r>=t} dt_r reverse."""
    u = np.asarray(u, np.float64)
    b, d, L = u.shape
    N = A.shape[1]
    dt = _dt_numpy(np.asarray(delta, np.float64), delta_bias, softplus)  # [b,d,L]
    S = np.cumsum(dt, axis=-1)  # S_t = sum_{r<=t} dt_r
    y = np.zeros((b, d, L))
    t_idx = np.arange(L)
    for bi in range(b):
        for di in range(d):
            St = S[bi, di]
            if not reverse:
                # exponent sum_{r=s+1..t} dt_r = S_t - S_s, valid for s <= t
                seg = St[:, None] - St[None, :]
                mask = t_idx[None, :] <= t_idx[:, None]
            else:
                # exponent sum_{r=t..s-1} dt_r = S_{s-1} - S_{t-1} = (S_s - dt_s) - (S_t - dt_t)
                Sm = St - dt[bi, di]
                seg = Sm[None, :] - Sm[:, None]
                mask = t_idx[None, :] >= t_idx[:, None]
            seg = np.where(mask, seg, 0.0)
            # K[t, s] = sum_n C[n,t] exp(A_n seg[t,s]) dt_s B[n,s]
            E = np.exp(A[di][:, None, None] * seg[None, :, :])  # [N, L, L]
            K = np.einsum("nt,nts,ns->ts", C[bi], E, B[bi]) * dt[bi, di][None, :]
            K = np.where(mask, K, 0.0)
            y[bi, di] = K @ u[bi, di] + (0.0 if D is None else D[di]) * u[bi, di]
            if h0 is not None:
                E = St if not reverse else St[-1] - St + dt[bi, di]
                y[bi, di] += np.einsum("nt,nt,n->t", C[bi], np.exp(A[di][:, None] * E[None, :]), h0[bi, di])
    return y


def brute_last_state(u, delta, A, B, delta_bias=None, softplus=True, reverse=False, h0=None):
    """State after the last scanned token, [b, d, N], as one weighted sum:
    h_n = exp(A_n sum_all dt) h0_n + sum_s exp(A_n W_s) dt_s B[n,s] u_s with
    W_s = sum of the step sizes scanned after token s (r > s forward, r < s reverse)."""
    u = np.asarray(u, np.float64)
    b, d, L = u.shape
    N = A.shape[1]
    dt = _dt_numpy(np.asarray(delta, np.float64), delta_bias, softplus)
    total = dt.sum(-1)  # [b, d]
    incl = np.cumsum(dt, -1)
    W = (total[..., None] - incl) if not reverse else (incl - dt)
    h = np.einsum("dn,bdns,bds,bns,bds->bdn", np.ones((d, N)), np.exp(A[None, :, :, None] * W[:, :, None, :]),
                  dt, B, u)
    if h0 is not None:
        h = h + np.exp(A[None] * total[..., None]) * h0
    return h


def silu_numpy(x):
    return x / (1.0 + np.exp(-x))


def brute(u, z, dirs, softplus=True, reverse_single=False):
    """Gated output; ``dirs`` holds one (forward, or reverse if ``reverse_single``)
    or two (forward, reverse) parameter dicts with delta, A, B, C, D, delta_bias."""
    if len(dirs) == 1:
        y = brute_dir(u, softplus=softplus, reverse=reverse_single, **dirs[0])
    else:
        y = brute_dir(u, softplus=softplus, reverse=False, **dirs[0]) + \
            brute_dir(u, softplus=softplus, reverse=True, **dirs[1])
    return y if z is None else y * silu_numpy(np.asarray(z, np.float64))


def brute_mp(u, z, dirs, softplus=True, reverse_single=False, dps=50):
    """Same sums as ``brute`` evaluated in mpmath with ``dps`` decimal digits.
    Returns a nested list of mpf values [b][d][t]."""
    import mpmath as mp

    mp.mp.dps = dps
    u = np.asarray(u, np.float64)
    b, d, L = u.shape

    def dir_out(p, reverse):
        A, B, C = p["A"], p["B"], p["C"]
        N = A.shape[1]
        D = p.get("D")
        bias = p.get("delta_bias")
        out = [[[mp.mpf(0)] * L for _ in range(d)] for _ in range(b)]
        for bi in range(b):
            for di in range(d):
                xs = [mp.mpf(float(p["delta"][bi, di, t])) + (mp.mpf(float(bias[di])) if bias is not None else 0)
                      for t in range(L)]
                dts = [mp.log1p(mp.exp(x)) if softplus else x for x in xs]
                for t in range(L):
                    acc = mp.mpf(0)
                    srange = range(0, t + 1) if not reverse else range(t, L)
                    for s in srange:
                        seg = (mp.fsum(dts[s + 1:t + 1]) if not reverse else mp.fsum(dts[t:s]))
                        kts = mp.mpf(0)
                        for n in range(N):
                            kts += mp.mpf(float(C[bi, n, t])) * mp.exp(mp.mpf(float(A[di, n])) * seg) \
                                * mp.mpf(float(B[bi, n, s]))
                        acc += kts * dts[s] * mp.mpf(float(u[bi, di, s]))
                    if D is not None:
                        acc += mp.mpf(float(D[di])) * mp.mpf(float(u[bi, di, t]))
                    out[bi][di][t] = acc
        return out

    if len(dirs) == 1:
        y = dir_out(dirs[0], reverse_single)
    else:
        yf, yr = dir_out(dirs[0], False), dir_out(dirs[1], True)
        y = [[[yf[i][j][t] + yr[i][j][t] for t in range(L)] for j in range(d)] for i in range(b)]
    if z is not None:
        for bi in range(b):
            for di in range(d):
                for t in range(L):
                    zz = mp.mpf(float(z[bi, di, t]))
                    y[bi][di][t] *= zz / (1 + mp.exp(-zz))
    return y
