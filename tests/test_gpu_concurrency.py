"""Calls made at the same time, from several host threads on streams of their own,
give the same bits as the same calls made one after another on one stream.

The library keeps no mutable state between calls (each call's scratch is the
caller's workspace) and its kernels are deterministic, so any difference would be a
race in the host code or a kernel reading another call's memory.  ctypes releases
the GIL for the duration of each C call, so the threads' launches really overlap.
"""
import threading

import pytest
import torch

from selective_state_space_sscan_amd import inputs as I
from selective_state_space_sscan_amd import sscan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPEATS = 4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    sscan.load_library()  # raises if the extension is missing: no fallback


def _jobs():
    """Four calls of different entry points and plans, inputs resident on the device.
    Each job returns its results as a tuple of tensors (fresh outputs each call)."""
    jobs = []

    # a segmented one-direction forward (aggregate, carry and output kernels)
    xs = I.make_inputs(2, 192, 5000, io_dtype="bf16", bc_dtype="f32", seed=11).to(DEV)
    ws = torch.empty(max(sscan.workspace_bytes(2, 192, 5000), 1), dtype=torch.uint8, device=DEV)
    jobs.append(lambda: (sscan.run_inputs(xs, workspace=ws),))

    # a short bidirectional forward (one segment per row)
    xb = I.make_inputs(4, 128, 197, bidir=True, io_dtype="f32", bc_dtype="f32", seed=12).to(DEV)
    wb = torch.empty(max(sscan.workspace_bytes(4, 128, 197, bidir=True), 1), dtype=torch.uint8, device=DEV)
    jobs.append(lambda: (sscan.run_inputs(xb, workspace=wb),))

    # a backward with the gate
    xg = I.make_inputs(1, 64, 3000, io_dtype="f32", bc_dtype="f32", seed=13).to(DEV)
    g = torch.randn(1, 64, 3000, generator=torch.Generator().manual_seed(13)).to(DEV)
    pg = xg.dirs[0]

    def backward():
        r = sscan.bwd(xg.u, xg.delta, pg.A, pg.B, pg.C, g, D=pg.D, z=xg.z, delta_bias=pg.delta_bias)
        return tuple(r[k] for k in ("du", "dz", "ddelta", "ddelta_bias", "dA", "dB", "dC", "dD"))
    jobs.append(backward)

    # the four-direction cross order of a small map (gathers, transposes, put-back)
    h, w = 24, 40
    x1 = I.make_inputs(2, 64, h * w, bidir=True, io_dtype="bf16", bc_dtype="bf16", seed=14).to(DEV)
    x2 = I.make_inputs(2, 64, h * w, bidir=True, io_dtype="bf16", bc_dtype="bf16", seed=15).to(DEV)
    dirs = [dict(delta=x1.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D) for p in x1.dirs + x2.dirs]
    kinds = [sscan.ORDER_ROW, sscan.ORDER_ROW_REV, sscan.ORDER_COL, sscan.ORDER_COL_REV]
    jobs.append(lambda: (sscan.multi(x1.u, x1.z, dirs, kinds, h, w),))
    return jobs


def test_concurrent_streams_and_threads_match_serial_calls():
    jobs = _jobs()
    ref = [job() for job in jobs]  # one after another, on the current stream
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in jobs]  # default priority
    results = [[None] * REPEATS for _ in jobs]
    errors = []
    start = threading.Barrier(len(jobs))

    def worker(k):
        try:
            with torch.cuda.stream(streams[k]):
                start.wait()
                for r in range(REPEATS):
                    results[k][r] = jobs[k]()
            streams[k].synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for k, per_job in enumerate(results):
        for r, got in enumerate(per_job):
            assert len(got) == len(ref[k])
            for i, (a, b) in enumerate(zip(got, ref[k])):
                if b is None:
                    assert a is None
                    continue
                assert torch.equal(a, b), (k, r, i)
