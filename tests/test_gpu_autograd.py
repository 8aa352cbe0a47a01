"""The autograd wrappers of the binding (``selective_scan``, ``selective_scan_bidir``):
torch.autograd through them gives exactly the backward entry points' gradients
(bitwise: the same kernels on the same inputs), and those match the fp64 oracle
(the backward's parity is tested in test_gpu_bwd.py; one case here closes the loop).
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from parity import TOL, metrics
from selective_state_space_sscan_amd import inputs as I
from selective_state_space_sscan_amd import sscan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def leaf(t):
    return t.detach().clone().to(DEV).requires_grad_(True)


@pytest.mark.parametrize("io,reverse", [("f32", False), ("bf16", True)])
def test_selective_scan_grads_are_the_backward_entry_point(io, reverse):
    x = I.make_inputs(2, 70, 300, io_dtype=io, bc_dtype=io, seed=77 + reverse)
    p = x.dirs[0]
    args = [leaf(t) for t in (x.u, x.delta, p.A, p.B, p.C, p.D, x.z, p.delta_bias)]
    g = torch.from_numpy(np.random.default_rng(5).standard_normal(tuple(x.u.shape), dtype=np.float32))
    g = g.to(x.u.dtype).to(DEV)
    y = sscan.selective_scan(*args, reverse=reverse)
    torch.autograd.backward(y, g)
    u, delta, A, B, C, D, z, bias = (a.detach() for a in args)
    ref = sscan.bwd(u, delta, A, B, C, g, D=D, z=z, delta_bias=bias, reverse=reverse)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), sscan.fwd(u, delta, A, B, C, D, z, bias, reverse=reverse))
    names = ["du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias"]
    for a, n in zip(args, names):
        assert torch.equal(a.grad, ref[n]), n
    # and the oracle, for du (the rest as in the backward's own parity tests)
    x64 = I.as_f64_dict(x)
    q = x64["dirs"][0]
    o = oracle.sscan_bwd(x64["u"], x64["z"], I.f64(g.cpu()), [dict(delta=x64["delta"], **q)], reverse=reverse)
    m = metrics(I.f64(args[0].grad.cpu()), o["du"])
    assert m["floored_max"] <= TOL[io], m


def test_selective_scan_bidir_shared_delta_gets_both_gradients():
    """One delta tensor for both directions: autograd adds the two directions'
    ddelta, as the pages' shared projection would need."""
    x = I.make_inputs(2, 64, 200, bidir=True, seed=81)
    pf, pr = x.dirs
    u, z, delta = leaf(x.u), leaf(x.z), leaf(x.delta)
    fp = {k: leaf(getattr(pf, k)) for k in ("A", "B", "C", "D", "delta_bias")}
    rp = {k: leaf(getattr(pr, k)) for k in ("A", "B", "C", "D", "delta_bias")}
    g = torch.randn(x.u.shape, generator=torch.Generator().manual_seed(3)).to(DEV)
    y = sscan.selective_scan_bidir(u, z, dict(fp, delta=delta), dict(rp, delta=delta))
    torch.autograd.backward(y, g)
    d = lambda m: {k: v.detach() for k, v in m.items()}
    ref = sscan.bidir_bwd(u.detach(), z.detach(), g, dict(d(fp), delta=delta.detach()), dict(d(rp), delta=delta.detach()))
    torch.cuda.synchronize()
    assert torch.equal(u.grad, ref["du"]) and torch.equal(z.grad, ref["dz"])
    assert torch.equal(delta.grad, ref["fwd"]["ddelta"] + ref["rev"]["ddelta"])
    for name, side, key in (("A", "fwd", "dA"), ("B", "fwd", "dB"), ("C", "rev", "dC"), ("D", "rev", "dD")):
        src = fp if side == "fwd" else rp
        assert torch.equal(src[name].grad, ref[side][key]), (side, name)
