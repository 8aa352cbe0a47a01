#!/usr/bin/env python3
"""Benchmark of the MI355X selective scan (Mamba S6) on one GPU.

Workload: the long-sequence single-direction scan (batch 1, d_inner 1536,
len 262144, dstate 16, bf16 u/delta/z/y, f32 B/C, seeded synthetic inputs already
resident in HBM).  One step = one sscan_fwd call (all its kernels).  Prints ONE
JSON line on stdout.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                 [--copy-calibration]

Timing: K plain calls between two HIP events give ms_per_step; K more calls of the
profiled entry point (events recorded between the call's kernels on the same
stream) give each kernel's average duration, and the dominant kernel's roofline.
--copy-calibration ends with a plain streaming kernel (negation of 512 MiB: 512 MiB
read, 512 MiB written), the known-size
reference that scales the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc
run of this command (selective_state_space_sscan_amd/profiling.py turns such runs
into profiles/traffic_<workload>.json, which fills "traffic" while the kernel
source is unchanged).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "selective-scan Melem/s (batch·dim·len) + achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9  # CUs x SIMDs x lanes x clock: non-packed fp32 lane-instructions/s
EXP_SLOTS = 2.0                 # v_exp_f32 issue cost in VALU slots (measured: half the FMA rate)
FLOPS_PER_ELEM_STATE = 6.0      # dt*A (1) + dt*u*B (1) + state FMA (2) + readout FMA (2)
SLOTS_PER_ELEM_STATE = 4.0 + EXP_SLOTS  # the same four VALU ops plus one exp
ALU_PEAK_TFLOPS = VALU_LANE_OPS / SLOTS_PER_ELEM_STATE * FLOPS_PER_ELEM_STATE / 1e12


def alg_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one call: u, delta, z read once, y written once,
    B and C read once per direction, A/D/bias per direction."""
    io = 2 if cfg.io_dtype == "bf16" else 4
    bc = 2 if cfg.bc_dtype == "bf16" else 4
    per_dir = 2 * cfg.batch * cfg.dstate * cfg.len * bc + cfg.dim * (cfg.dstate + 2) * 4
    return 4 * cfg.elems * io + cfg.ndir * per_dir


def cpu_baseline(x, y_gpu, cfg, target_s: float = 8.0):
    """The fp64 oracle, as it stands, on whole sampled rows of the same inputs,
    using every host core available to this process."""
    import numpy as np

    from oracle import oracle
    from selective_state_space_sscan_amd import inputs as I

    cores = oracle.default_threads()

    def run_rows(rows):
        out = []
        for b, d in rows:
            sl = lambda t: I.f64(t[b:b + 1, d:d + 1])
            u, z, delta = sl(x.u), sl(x.z), sl(x.delta)
            ps = [dict(delta=delta, A=I.f64(p.A[d:d + 1]), B=I.f64(p.B[b:b + 1]), C=I.f64(p.C[b:b + 1]),
                       D=I.f64(p.D[d:d + 1]), delta_bias=I.f64(p.delta_bias[d:d + 1])) for p in x.dirs]
            if len(ps) == 1:
                p = ps[0]
                out.append(oracle.sscan_fwd(u, delta, p["A"], p["B"], p["C"], p["D"], z, p["delta_bias"], nthreads=1))
            else:
                out.append(oracle.sscan_bidir(u, z, ps[0], ps[1], nthreads=1))
        return out

    # rows are independent: run them on all cores with a thread pool (the C oracle
    # releases the GIL inside ctypes calls)
    from concurrent.futures import ThreadPoolExecutor

    rng = np.random.default_rng(1234)
    all_rows = [(b, d) for b in range(cfg.batch) for d in range(cfg.dim)]
    order = [all_rows[i] for i in rng.permutation(len(all_rows))]
    # calibrate on one row per core, then size the sample to about target_s
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(lambda r: run_rows([r]), order[:cores]))
    t_cal = time.perf_counter() - t0
    n_rows = int(min(len(order), max(cores, cores * target_s / max(t_cal, 1e-6))))
    sample = order[:n_rows]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        refs = list(ex.map(lambda r: run_rows([r])[0], sample))
    dt = time.perf_counter() - t0
    elems = n_rows * cfg.len
    # parity of the GPU output on the same sampled rows (the oracle output is at hand)
    got = np.concatenate([I.f64(y_gpu[b:b + 1, d:d + 1].cpu()) for b, d in sample[:64]], 1)
    ref = np.concatenate(refs[:64], 1)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref) / (np.abs(ref) + rms)))
    return {
        "value": elems / dt / 1e6, "unit": "Melem/s", "cores": cores, "kind": "oracle",
        "sample": f"{n_rows} whole rows of {cfg.len} tokens ({elems} elements, {cfg.ndir} direction(s)) "
                  f"of the same seeded inputs, fp64 sequential per row, {cores} threads, {dt:.1f} s",
        "seconds": dt, "gpu_parity_on_sample": {"floored_max_err": err, "rows_compared": min(64, n_rows)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long-seq-fwd")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with a 512 MiB negation kernel (counter calibration for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        sys.exit("bench.py measures one GPU only: this build has no multi-GPU path "
                 "(run with --gpus 1)")

    import torch

    from selective_state_space_sscan_amd import inputs as I
    from selective_state_space_sscan_amd import sscan

    sscan.load_library()
    names = [c.name for c in I.CONFIGS]
    ci = names.index(args.workload)
    cfg = I.CONFIGS[ci]
    dev = torch.device("cuda:0")
    x = I.config_inputs(ci, 0)
    xd = x.to(dev)
    ws_bytes = sscan.workspace_bytes(cfg.batch, cfg.dim, cfg.len, cfg.dstate, cfg.bidir)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    y = torch.empty_like(xd.u)

    def step(events=None):
        sscan.run_inputs(xd, out=y, workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    value = cfg.elems / (ms * 1e-3) / 1e6
    # per-kernel timing: the profiled entry point records HIP events between the
    # call's kernels on the same stream (one event set per call)
    evsets = [sscan.HipEvents() for _ in range(args.steps)]
    for k in range(args.steps):
        step(evsets[k])
    torch.cuda.synchronize()
    per_kernel = {name: [] for name in sscan.PROFILE_STEPS}
    for ev in evsets:
        for name, v in ev.step_ms().items():
            per_kernel[name].append(v)
    kernel_ms = {name: sum(v) / len(v) for name, v in per_kernel.items()}
    dominant = max(kernel_ms, key=kernel_ms.get)
    if args.copy_calibration:
        # a plain streaming kernel of known traffic: reads 512 MiB, writes 512 MiB
        src = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    nbytes = alg_bytes(cfg)
    # algorithmic work of the output kernel: the full recurrence and readout of
    # every element and direction (it also moves every algorithmic byte)
    flops = FLOPS_PER_ELEM_STATE * cfg.dstate * cfg.elems * cfg.ndir
    t_dom = kernel_ms[dominant] * 1e-3
    achieved_tflops = flops / t_dom / 1e12
    out = {
        "metric": METRIC, "value": value, "unit": "Melem/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded numpy PCG64, shapes of the pages' workloads)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "dim": cfg.dim, "len": cfg.len, "dstate": cfg.dstate,
                   "directions": cfg.ndir, "io_dtype": cfg.io_dtype, "bc_dtype": cfg.bc_dtype},
        "roofline": {"bound": "alu", "kernel": dominant, "achieved": achieved_tflops, "peak": ALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved_tflops / ALU_PEAK_TFLOPS, "traffic": None},
        "kernels_ms": kernel_ms,
        "step_alu": {"achieved_TFLOPs": flops / (ms * 1e-3) / 1e12,
                     "frac": flops / (ms * 1e-3) / 1e12 / ALU_PEAK_TFLOPS},
        "hbm": {"achieved_GBs": nbytes / (ms * 1e-3) / 1e9, "peak_GBs": HBM_PEAK_GBS,
                "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes_per_step": nbytes},
        "wall_s_timed": wall,
    }
    if dominant != "output":
        out["roofline"]["kernel"] = dominant
    from selective_state_space_sscan_amd import profiling

    traffic = profiling.load_traffic(os.path.join(ROOT, "profiles", f"traffic_{cfg.name}.json"))
    if traffic and dominant in traffic["per_launch"]:
        out["roofline"]["traffic"] = traffic["per_launch"][dominant]["bytes"]
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(x, y, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
