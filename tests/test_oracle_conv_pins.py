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
