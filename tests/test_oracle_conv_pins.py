"""Pins of the fp64 depthwise convolution in front of the scan (oracle/sscan_oracle_conv.c).

Checked against library routines it shares nothing with (numpy.convolve, PyTorch's
grouped conv1d) and against the impulse response.  No HIP code is involved.
"""
import numpy as np
import pytest
import torch

from oracle import oracle


@pytest.mark.parametrize("width", [1, 2, 3, 4])
def test_causal_matches_numpy_convolve(width):
    """Causal cross-correlation = numpy's convolution with the reversed kernel,
    cut to the first len outputs (Mamba2 page, section 4.4: padding d_conv - 1,
    then [:L]).  Catches a flipped kernel, an off-by-one shift, right padding."""
    rng = np.random.default_rng(width)
    b, d, L = 2, 3, 17
    x = rng.normal(size=(b, d, L))
    w = rng.normal(size=(d, width))
    bias = rng.normal(size=d)
    out = oracle.conv1d(x, w, bias)
    for bi in range(b):
        for di in range(d):
            ref = np.convolve(x[bi, di], w[di, ::-1])[:L] + bias[di]
            np.testing.assert_allclose(out[bi, di], ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("width,same", [(4, False), (3, False), (3, True), (1, True)])
def test_matches_torch_grouped_conv1d(width, same):
    """The layers on the pages: nn.Conv1d(groups=d_inner) with padding d_conv - 1
    and the output cut to L (causal), or padding (k - 1) / 2 (same)."""
    rng = np.random.default_rng(10 + width)
    b, d, L = 2, 5, 23
    x = rng.normal(size=(b, d, L))
    w = rng.normal(size=(d, width))
    bias = rng.normal(size=d)
    pad = (width - 1) // 2 if same else width - 1
    ref = torch.nn.functional.conv1d(torch.tensor(x), torch.tensor(w)[:, None, :], torch.tensor(bias), padding=pad,
                                     groups=d)[:, :, :L].numpy()
    np.testing.assert_allclose(oracle.conv1d(x, w, bias, same=same), ref, rtol=1e-13, atol=1e-13)
    silu_ref = ref / (1.0 + np.exp(-ref))
    np.testing.assert_allclose(oracle.conv1d(x, w, bias, same=same, silu=True), silu_ref, rtol=1e-13, atol=1e-13)


def test_impulse_response_and_edges():
    """A unit impulse at t0 reproduces the kernel taps after it (causal) or centred
    on it (same); zeros come in from both ends of the sequence."""
    d, L, t0 = 2, 12, 5
    w = np.array([[1.0, 2.0, 3.0, 4.0], [0.5, -1.0, 2.0, 0.25]])
    x = np.zeros((1, d, L))
    x[0, :, t0] = 1.0
    out = oracle.conv1d(x, w)
    for di in range(d):
        ref = np.zeros(L)
        ref[t0:t0 + 4] = w[di, ::-1]
        np.testing.assert_array_equal(out[0, di], ref)
    w3 = w[:, :3]
    out = oracle.conv1d(x, w3, same=True)
    for di in range(d):
        ref = np.zeros(L)
        ref[t0 - 1:t0 + 2] = w3[di, ::-1]
        np.testing.assert_array_equal(out[0, di], ref)
    with pytest.raises(RuntimeError):
        oracle.conv1d(x, w, same=True)  # even width has no centred 'same'


# --- the decode step through the convolution (oracle.sscan_step_conv) ---------------------------

def _decode_case(seed, b=2, d=5, L=13, width=4, silu=True):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(b, d, L))
    delta = 0.5 * rng.normal(size=(b, d, L))
    z = rng.normal(size=(b, d, L))
    A = -np.exp(rng.uniform(-1.0, 1.5, size=(d, 16)))
    B = rng.normal(size=(b, 16, L))
    C = rng.normal(size=(b, 16, L))
    D = rng.normal(size=d)
    bias = np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=d))))
    w = rng.normal(0.0, 0.5, size=(d, width))
    wb = rng.normal(0.0, 0.2, size=d)
    return x, delta, z, A, B, C, D, bias, w, wb


@pytest.mark.parametrize("width,silu", [(4, True), (3, False), (2, True), (1, False)])
def test_decode_steps_equal_the_sequence_call(width, silu):
    """Token-by-token steps from zero states (zero state = the causal padding)
    reproduce the fused sequence call's outputs, its final scan state, and leave
    the last width - 1 inputs in the convolution state."""
    x, delta, z, A, B, C, D, bias, w, wb = _decode_case(20 + width, width=width, silu=silu)
    b, d, L = x.shape
    ref = oracle.sscan_fwd_conv(x, w, wb, False, silu, delta, A, B, C, D, z, bias)
    u = oracle.conv1d(x, w, wb, same=False, silu=silu)
    _, ref_h = oracle.sscan_fwd(u, delta, A, B, C, D, z, bias, return_last_state=True)
    h = np.zeros((b, d, 16))
    cs = np.zeros((b, d, width - 1))
    ys = []
    for t in range(L):
        y, h, cs = oracle.sscan_step_conv(h, cs, x[:, :, t], w, wb, silu, delta[:, :, t], A, B[:, :, t], C[:, :, t],
                                          D, z[:, :, t], bias)
        ys.append(y)
    np.testing.assert_allclose(np.stack(ys, -1), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h, ref_h, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(cs, x[:, :, L - (width - 1):] if width > 1 else np.zeros((b, d, 0)))


def test_decode_conv_state_is_the_input_history():
    """A nonzero convolution state acts as the inputs before the first step: the
    step outputs equal the sequence call on [history, x] at x's positions, with the
    scan state taken over history first."""
    width = 4
    x, delta, z, A, B, C, D, bias, w, wb = _decode_case(31, L=9, width=width)
    b, d, L = x.shape
    rng = np.random.default_rng(32)
    hist = rng.normal(size=(b, d, width - 1))
    h0 = rng.normal(size=(b, d, 16))
    # the convolved sequence over [history, x], restricted to x's positions
    u_full = oracle.conv1d(np.concatenate([hist, x], 2), w, wb, same=False, silu=True)[:, :, width - 1:]
    ref = oracle.sscan_fwd(u_full, delta, A, B, C, D, z, bias, h0=h0)
    h, cs, ys = h0, hist, []
    for t in range(L):
        y, h, cs = oracle.sscan_step_conv(h, cs, x[:, :, t], w, wb, True, delta[:, :, t], A, B[:, :, t], C[:, :, t],
                                          D, z[:, :, t], bias)
        ys.append(y)
    np.testing.assert_allclose(np.stack(ys, -1), ref, rtol=1e-12, atol=1e-12)


# --- the backward through the convolution (oracle.conv1d_bwd, oracle.sscan_bwd_conv) -----------

@pytest.mark.parametrize("width,same,silu", [(4, False, True), (3, False, False), (3, True, True), (1, True, False),
                                             (2, False, True)])
def test_conv1d_bwd_matches_torch_autograd(width, same, silu):
    """PyTorch's reverse mode (a library routine) through its grouped conv1d with the
    pages' paddings, cut to L, and silu."""
    rng = np.random.default_rng(40 + width + 7 * same)
    b, d, L = 2, 5, 19
    x = rng.normal(size=(b, d, L))
    w = rng.normal(size=(d, width))
    bias = rng.normal(size=d)
    g = rng.normal(size=(b, d, L))
    dx, dw, db = oracle.conv1d_bwd(x, w, bias, same, silu, g)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    xt, wt, bt = T(x), T(w), T(bias)
    pad = (width - 1) // 2 if same else width - 1
    out = torch.nn.functional.conv1d(xt, wt[:, None, :], bt, padding=pad, groups=d)[:, :, :L]
    if silu:
        out = torch.nn.functional.silu(out)
    (out * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def _fused_loss(x, w, wb, same, silu, z, g, dirs, reverse):
    if len(dirs) == 1:
        p = dirs[0]
        y = oracle.sscan_fwd_conv(x, w, wb, same, silu, p["delta"], p["A"], p["B"], p["C"], p["D"], z,
                                  p["delta_bias"], reverse=reverse)
    else:
        u = oracle.conv1d(x, w, wb, same, silu)
        y = oracle.sscan_bidir(u, z, dirs[0], dirs[1])
    return float(np.sum(g * y))


@pytest.mark.parametrize("ndir,width,same,silu,reverse", [(1, 4, False, True, False), (1, 3, False, False, True),
                                                          (2, 3, True, True, False)])
def test_sscan_bwd_conv_matches_central_differences(ndir, width, same, silu, reverse):
    """dx, dconv_w, dconv_b and a parameter gradient of the fused backward against
    central differences of the fused forward oracle (the convolution's output feeds
    the scan as u; its pins and the scan's are separate)."""
    rng = np.random.default_rng(60 + ndir + width)
    b, d, L = 2, 3, 10
    x = rng.normal(size=(b, d, L))
    z = rng.normal(size=(b, d, L))
    g = rng.normal(size=(b, d, L))
    w = rng.normal(0.0, 0.5, size=(d, width))
    wb = rng.normal(0.0, 0.2, size=d)
    dirs = [dict(delta=rng.normal(0.0, 0.5, (b, d, L)), A=-np.exp(rng.uniform(-1.0, 1.5, (d, 16))),
                 B=rng.normal(size=(b, 16, L)), C=rng.normal(size=(b, 16, L)), D=rng.normal(size=d),
                 delta_bias=rng.uniform(-3.0, 0.5, d)) for _ in range(ndir)]
    got = oracle.sscan_bwd_conv(x, w, wb, same, silu, z, g, dirs, reverse=reverse)
    h = 1e-5

    def loss(args):
        xx, ww, bb, dd = args
        return _fused_loss(xx, ww, bb, same, silu, z, g, dd, reverse)

    def central(mutate):
        return (loss(mutate(h)) - loss(mutate(-h))) / (2 * h)

    checks = []
    for idx in [(0, 0, 0), (1, 2, 9), (0, 1, 5), (1, 0, L - 2)]:
        def mx(e, idx=idx):
            xx = x.copy()
            xx[idx] += e
            return xx, w, wb, dirs
        checks.append(("dx", got["dx"][idx], central(mx)))
    for idx in [(0, 0), (2, width - 1), (1, width // 2)]:
        def mw(e, idx=idx):
            ww = w.copy()
            ww[idx] += e
            return x, ww, wb, dirs
        checks.append(("dconv_w", got["dconv_w"][idx], central(mw)))
    for i in range(d):
        def mb(e, i=i):
            bb = wb.copy()
            bb[i] += e
            return x, w, bb, dirs
        checks.append(("dconv_b", got["dconv_b"][i], central(mb)))
    def md(e):
        nd = [dict(p) for p in dirs]
        arr = nd[0]["delta"].copy()
        arr[1, 1, 3] += e
        nd[0]["delta"] = arr
        return x, w, wb, nd
    checks.append(("ddelta", got["dirs"][0]["ddelta"][1, 1, 3], central(md)))
    for name, val, ref in checks:
        assert abs(val - ref) <= 1e-6 * (1.0 + abs(ref)), (name, val, ref)
