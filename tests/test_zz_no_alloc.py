"""sscan_fwd_noalloc (the entry point for callers that cannot allocate) against
sscan_fwd, through the C ABI: two calls in a row on one GPU, the second with a
smaller input, each equal to sscan_fwd on the same inputs (same kernels: bitwise)
and within the float32 / bfloat16 bound of the oracle."""
import os

import pytest
import torch

from oracle import oracle
from parity import TOL, metrics
from selective_state_space_sscan_amd import inputs as I
from selective_state_space_sscan_amd import sscan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SCRATCH_BYTES = sscan.NOALLOC_SCRATCH_BYTES


def noalloc_fwd(xd, reverse=False):
    p = xd.dirs[0]
    return sscan.fwd_noalloc(xd.u, xd.delta, p.A, p.B, p.C, p.D, xd.z, p.delta_bias, reverse=reverse)


@pytest.mark.parametrize("reverse", [False, True])
def test_noalloc_matches_fwd_two_calls(reverse):
    if not os.path.exists(oracle.LIB):
        oracle.build(force=True)
    cases = [(2, 192, 20000, "bf16", "f32"), (1, 70, 1000, "f32", "f32")]  # second: smaller
    for k, (b, d, L, io, bc) in enumerate(cases):
        x = I.make_inputs(b, d, L, io_dtype=io, bc_dtype=bc, seed=4100 + k + 10 * reverse)
        need = sscan.workspace_bytes(b, d, L)
        assert 0 < need <= SCRATCH_BYTES
        xd = x.to(DEV)
        y_na = noalloc_fwd(xd, reverse)
        p = xd.dirs[0]
        y_ref = sscan.fwd(xd.u, xd.delta, p.A, p.B, p.C, p.D, xd.z, p.delta_bias, reverse=reverse)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16 if io == "bf16" else torch.int32),
                           y_ref.view(torch.int16 if io == "bf16" else torch.int32)), (k, reverse)
        ref = oracle.run_inputs(I.as_f64_dict(x), nthreads=min(16, oracle.default_threads()), reverse=reverse)
        m = metrics(I.f64(y_na.cpu()), ref)
        print(f"noalloc call {k} reverse={reverse} {b}x{d}x{L} {io}: {m}", flush=True)
        assert m["floored_max"] <= TOL[io]
