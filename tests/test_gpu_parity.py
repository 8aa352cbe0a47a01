"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case draws seeded inputs, runs ``libsscan.so`` on cuda:0 and compares with
the oracle on the same (exactly widened) values using the floored relative error
of tests/parity.py: <= 1e-4 for float32 I/O, <= 2e-2 for bfloat16 I/O.
The five workloads are compared in full (every channel and token), with A as the
workloads' recipe gives it (S4D-real, the same for every channel) and with A drawn
per (channel, state) (A = -exp(A_log)); the long-sequence workload in the launch
configuration the benchmark times.  The edge cases draw A per (channel, state).
"""
import os
import zlib

import numpy as np
import pytest
import torch

from oracle import oracle
from parity import TOL, metrics
from selective_state_space_sscan_amd import inputs as I
from selective_state_space_sscan_amd import sscan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NTHREADS = min(16, oracle.default_threads())


@pytest.fixture(scope="module", autouse=True)
def _lib():
    sscan.load_library()  # raises if the extension is missing: no fallback
    if not os.path.exists(oracle.LIB):
        oracle.build(force=True)


def gpu_run(x, softplus=True, gate=True, reverse=False):
    xd = x.to(DEV)
    z = xd.z if gate else None
    if len(xd.dirs) == 1:
        p = xd.dirs[0]
        y = sscan.fwd(xd.u, xd.delta, p.A, p.B, p.C, p.D, z, p.delta_bias, softplus=softplus, reverse=reverse)
    else:
        mk = lambda p: dict(delta=xd.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D)
        y = sscan.bidir(xd.u, z, mk(xd.dirs[0]), mk(xd.dirs[1]), softplus=softplus)
    torch.cuda.synchronize()
    return y


def oracle_run(x, softplus=True, gate=True, reverse=False):
    return oracle.run_inputs(I.as_f64_dict(x), softplus=softplus, nthreads=NTHREADS, reverse=reverse, gate=gate)


def check(got, ref, io_dtype, what):
    if isinstance(got, torch.Tensor):
        got = I.f64(got.cpu())
    m = metrics(got, ref)
    print(f"{what}: {m}", flush=True)
    assert m["floored_max"] <= TOL[io_dtype], (what, m)
    return m


@pytest.mark.parametrize("a_init", ["s4d", "random"])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_config_full_parity(cfg, a_init):
    x = I.config_inputs(cfg, 0, a_init=a_init)
    got = gpu_run(x)
    ref = oracle_run(x)
    check(got, ref, x.io_dtype, f"config {cfg} ({I.CONFIGS[cfg].name}) A {a_init}")


@pytest.mark.parametrize("cfg,k", [(0, 1), (0, 2), (1, 1), (1, 2), (2, 1), (2, 2), (3, 1), (3, 2)])
def test_configs_more_seeds(cfg, k):
    x = I.config_inputs(cfg, k)
    check(gpu_run(x), oracle_run(x), x.io_dtype, f"config {cfg} seed {k}")


def check_chunked(got, ref, io_dtype, what, rows_per_chunk=64):
    """check() for outputs too large to hold several float64 copies of: the RMS of
    the whole reference first, then the floored error chunk by chunk of channels."""
    b, d, L = ref.shape
    rms = float(np.sqrt(sum(float(np.sum(ref[:, i:i + rows_per_chunk] ** 2)) for i in range(0, d, rows_per_chunk))
                        / ref.size))
    worst, at = 0.0, None
    for i in range(0, d, rows_per_chunk):
        r = ref[:, i:i + rows_per_chunk]
        g = I.f64(got[:, i:i + rows_per_chunk])
        e = np.abs(g - r) / (np.abs(r) + rms)
        if not np.isfinite(g).all():
            worst, at = float("inf"), i
            break
        if e.max() > worst:
            worst, at = float(e.max()), i + int(np.unravel_index(np.argmax(e), e.shape)[1])
    print(f"{what}: floored max {worst:.3e} (channel {at}), rms {rms:.3e}", flush=True)
    assert worst <= TOL[io_dtype], (what, worst, at)


@pytest.mark.parametrize("k,a_init", [(0, "s4d"), (1, "s4d"), (2, "s4d"), (0, "random")])
def test_config4_long_sequence_full(k, a_init):
    """The benchmark's workload in the launch configuration it times (one row of
    1536 channels x 262144 tokens, 512 segments), every channel and token against
    the oracle."""
    x = I.config_inputs(4, k, a_init=a_init)
    got = gpu_run(x).cpu()
    ref = oracle_run(x)
    check_chunked(got, ref, "bf16", f"config 4 seed {k} A {a_init}, all 1536 channels")


def channel_rows(x, rows):
    """The oracle's fp64 inputs restricted to channels `rows` (B and C are per batch
    row and stay whole), sliced before widening."""
    sl = lambda t: I.f64(t[:, rows].contiguous())
    return dict(u=sl(x.u), delta=sl(x.delta), z=sl(x.z),
                dirs=[dict(A=I.f64(p.A[rows].contiguous()), B=I.f64(p.B), C=I.f64(p.C), D=I.f64(p.D[rows].contiguous()),
                           delta_bias=I.f64(p.delta_bias[rows].contiguous())) for p in x.dirs])


def test_bidir_long_aggregate_runs():
    """A 1M-token bidirectional scan: 16384 segments of 64 tokens, grouped in aggregate
    runs (sscan_scan_plan) so that the carry chains the runs and the output kernels
    rebuild each segment's entry state from its run; whole rows of sampled channels
    against the oracle."""
    b, d, L = 1, 64, 1 << 20
    assert sscan.scan_plan(b, d, L, bidir=True)["run_len"] > 1
    x = I.make_inputs(b, d, L, bidir=True, io_dtype="bf16", bc_dtype="bf16", seed=77, dt_range=(1e-4, 1e-2))
    got = gpu_run(x).cpu()
    rows = [0, 17, 63]
    ref = oracle_run_dict(channel_rows(x, rows))
    check(I.f64(got[:, rows]), ref, "bf16", f"1M-token bidirectional, rows {rows}")


def oracle_run_dict(x64):
    return oracle.run_inputs(x64, nthreads=NTHREADS)


EDGE = [
    # name, batch, dim, len, bidir, io, bc, kwargs
    ("len1-fwd", 2, 64, 1, False, "f32", "f32", {}),
    ("len1-bidir", 2, 64, 1, True, "f32", "f32", {}),
    ("len2-bidir", 1, 64, 2, True, "f32", "f32", {}),
    ("dim-tail-fwd", 2, 70, 45, False, "f32", "f32", {}),
    ("dim-tail-bidir", 3, 130, 33, True, "bf16", "bf16", {}),
    ("dim1", 1, 1, 100, True, "f32", "f32", {}),
    ("short-max", 2, 64, 256, True, "f32", "f32", {}),
    ("short-max+1", 2, 64, 257, True, "f32", "f32", {}),
    ("split-few-segments", 1, 64, 300, False, "f32", "f32", {}),
    ("split-few-segments-bidir", 1, 64, 300, True, "f32", "f32", {}),
    ("long-ragged-fwd", 2, 96, 1000, False, "f32", "f32", {}),
    ("long-ragged-rev", 2, 96, 1000, False, "f32", "f32", dict(reverse=True)),
    ("long-ragged-bidir", 2, 96, 1003, True, "f32", "f32", {}),
    ("long-bf16-f32bc", 1, 128, 5000, False, "bf16", "f32", {}),
    ("long-bf16-bidir", 1, 64, 4099, True, "bf16", "bf16", {}),
    ("no-gate", 2, 64, 300, True, "f32", "f32", dict(gate=False)),
    ("no-softplus", 2, 64, 50, False, "f32", "f32", dict(softplus=False)),
    ("rev-short", 2, 64, 50, False, "bf16", "bf16", dict(reverse=True)),
    # the one-direction bf16 output kernel (held to four waves per SIMD) in its
    # reverse and ungated instances, over several segments with a ragged end
    ("long-bf16-rev", 2, 64, 3001, False, "bf16", "bf16", dict(reverse=True)),
    ("long-bf16-no-gate", 1, 128, 2050, False, "bf16", "bf16", dict(gate=False)),
    # one-segment sequences of the four-lanes-per-channel kernel: 16-token tiles
    # (whole, one short of, one past), the two directions' meeting point (at 0 below
    # 32 tokens), channel counts that leave a wave's 16 channels partly idle
    ("quad-len15-bidir", 3, 16, 15, True, "f32", "f32", {}),
    ("quad-len16-bidir", 2, 32, 16, True, "bf16", "bf16", {}),
    ("quad-len17-fwd", 2, 48, 17, False, "f32", "f32", {}),
    ("quad-len33-bidir", 2, 37, 33, True, "f32", "f32", {}),
    ("quad-len100-rev", 3, 21, 100, False, "f32", "f32", dict(reverse=True)),
    ("quad-len197-bf16-rev", 2, 50, 197, False, "bf16", "f32", dict(reverse=True)),
    ("quad-len255-bidir-no-gate", 2, 40, 255, True, "bf16", "bf16", dict(gate=False)),
    ("quad-len64-bidir-no-softplus", 2, 24, 64, True, "f32", "f32", dict(softplus=False)),
]


@pytest.mark.parametrize("name,b,d,L,bidir,io,bc,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, b, d, L, bidir, io, bc, kw):
    x = I.make_inputs(b, d, L, bidir=bidir, io_dtype=io, bc_dtype=bc, seed=zlib.crc32(name.encode()) % 10000)
    if not kw.get("softplus", True):
        # without softplus the step is delta + bias itself: keep it positive
        x.delta.abs_().add_(0.01)
        for p in x.dirs:
            p.delta_bias.zero_()
    got = gpu_run(x, **kw)
    ref = oracle_run(x, **kw)
    check(got, ref, io, name)


def test_optional_D_and_bias_absent():
    x = I.make_inputs(2, 64, 300, seed=5)
    xd = x.to(DEV)
    p = xd.dirs[0]
    y = sscan.fwd(xd.u, xd.delta, p.A, p.B, p.C, None, xd.z, None)
    torch.cuda.synchronize()
    x64 = I.as_f64_dict(x)
    q = x64["dirs"][0]
    ref = oracle.sscan_fwd(x64["u"], x64["delta"], q["A"], q["B"], q["C"], None, x64["z"], None)
    check(y, ref, "f32", "no D, no bias")


def test_deterministic_reruns():
    x = I.config_inputs(3, 1).to(DEV)
    a = sscan.run_inputs(x)
    b = sscan.run_inputs(x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("L", [600, 150])
def test_nan_propagates_like_the_oracle(L):
    for bidir in (False, True):
        x = I.make_inputs(2, 64, L, bidir=bidir, seed=9)
        x.u[1, 5, L // 2 + 33] = float("nan")
        got = I.f64(gpu_run(x).cpu())
        ref = oracle_run(x)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), bidir
        fin = ~np.isnan(ref)
        m = metrics(got[fin], ref[fin])
        assert m["floored_max"] <= TOL["f32"]


def test_empty_input_returns_empty():
    u = torch.empty(2, 0, 5, device=DEV)
    A = torch.empty(0, 16, device=DEV)
    B = torch.randn(2, 16, 5, device=DEV)
    y = sscan.fwd(u, u, A, B, B)
    assert y.shape == (2, 0, 5)


def test_step_size_softplus_accuracy():
    """With len 1, B = C = 1/4 (sum_n C_n B_n = 1), no D and no gate, the output is
    the step size softplus(delta + bias) itself, so this pins the kernel's softplus
    (exp and log included) elementwise, including the small steps (down to about
    1e-13) that the long-memory workloads use."""
    d = 4096
    x = np.concatenate([np.linspace(-30.0, 30.0, d - 64), [0.0, 1e-7, -1e-7, 20.0, -20.0] + [-9.2] * 59])
    u = torch.ones(1, d, 1)
    delta = torch.tensor(x, dtype=torch.float32).view(1, d, 1)
    A = -torch.ones(d, 16)
    B = torch.full((1, 16, 1), 0.25)
    dev = lambda t: t.to(DEV).contiguous()
    y = sscan.fwd(dev(u), dev(delta), dev(A), dev(B), dev(B))
    torch.cuda.synchronize()
    got = I.f64(y.cpu()).ravel()
    ref = oracle.sscan_fwd(I.f64(u), I.f64(delta), I.f64(A), I.f64(B), I.f64(B)).ravel()
    rel = np.abs(got - ref) / np.abs(ref)
    print(f"softplus max rel err {rel.max():.3e} at x={x[np.argmax(rel)]:.4g}", flush=True)
    assert rel.max() <= 2e-6


DEGENERATE = [
    # A = 0: no decay, the state is the running sum of dt u B (Mamba2 page section
    # 2.2 with exp(0) = 1); several segments, so the carry chains plain sums
    ("A-zero", dict(A=0.0)),
    # dt -> 0 (softplus of a very negative input): the state never moves and the
    # output is D u alone, gated
    ("dt-to-zero", dict(delta=-60.0)),
    # very large steps (dt = 40): exp(dt A) is at most about 4e-7, so each token all
    # but forgets everything before it and y_t is close to dt_t u_t (C_t . B_t) + D u_t
    ("dt-large", dict(delta=40.0)),
]


@pytest.mark.parametrize("name,mod", DEGENERATE, ids=[d[0] for d in DEGENERATE])
@pytest.mark.parametrize("bidir", [False, True])
def test_degenerate_regimes(name, mod, bidir):
    """The method's degenerate regimes over segmented sequences (the aggregate and
    carry steps run): A = 0, dt -> 0, dt -> infinity."""
    x = I.make_inputs(2, 96, 3000, bidir=bidir, io_dtype="f32", bc_dtype="f32",
                      seed=zlib.crc32(name.encode()) % 10000 + int(bidir))
    if "A" in mod:
        for p in x.dirs:
            p.A.fill_(mod["A"])
    if "delta" in mod:
        x.delta.fill_(mod["delta"])
        for p in x.dirs:
            p.delta_bias.zero_()
    check(gpu_run(x), oracle_run(x), "f32", f"{name} bidir={bidir}")


# Whole-line loads.  Where bf16 rows and segments start on 128-byte lines, the
# one-direction output pass and the aggregate pass read u and delta a whole line
# (two tiles) at a time, the second tile by way of LDS.  The same inputs placed 16
# bytes past a line (16-byte vectors still, lines no longer) take the tile-at-a-time
# path.  Both runs are compared with the oracle, and with each other: the arithmetic
# is the same, so they agree bitwise.
LINE_CASES = [
    # name, batch, dim, len, kwargs
    ("fwd-segments", 2, 128, 4096, {}),
    ("rev-segments", 2, 128, 4096, dict(reverse=True)),
    ("no-gate", 1, 192, 2048, dict(gate=False)),
    ("one-segment", 4, 64, 192, {}),
    ("one-pair", 3, 64, 64, dict(reverse=True)),
    ("not-on-lines", 2, 64, 4096 + 32, {}),  # rows 64 bytes off a line: no pairs
]


def offset_copy(t, elems):
    """t copied into a buffer that starts `elems` elements past an allocation."""
    buf = torch.empty(t.numel() + elems, dtype=t.dtype, device=t.device)
    v = buf[elems:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("name,b,d,L,kw", LINE_CASES, ids=[c[0] for c in LINE_CASES])
def test_whole_line_loads(name, b, d, L, kw):
    x = I.make_inputs(b, d, L, io_dtype="bf16", bc_dtype="f32", seed=zlib.crc32(name.encode()) % 10000,
                      a_init="random")
    xd = x.to(DEV)
    p = xd.dirs[0]
    z = xd.z if kw.get("gate", True) else None
    rev = kw.get("reverse", False)
    assert xd.u.data_ptr() % 128 == 0 and xd.delta.data_ptr() % 128 == 0
    y_line = sscan.fwd(xd.u, xd.delta, p.A, p.B, p.C, p.D, z, p.delta_bias, reverse=rev)
    u8, d8 = offset_copy(xd.u, 8), offset_copy(xd.delta, 8)
    assert u8.data_ptr() % 128 == 16
    y_tile = sscan.fwd(u8, d8, p.A, p.B, p.C, p.D, z, p.delta_bias, reverse=rev)
    torch.cuda.synchronize()
    assert torch.equal(y_line, y_tile), f"{name}: whole-line and tile paths differ"
    ref = oracle_run(x, gate=kw.get("gate", True), reverse=rev)
    check(y_line, ref, "bf16", f"whole lines {name}")
