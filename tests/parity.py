"""Error metrics shared by the GPU parity tests and the benchmark's parity check.

err = max_i |yhat_i - y_i| / (|y_i| + rms(y)) over the compared outputs: an
elementwise relative error floored by the output's RMS, so that outputs near zero
(zeros of silu(z), cancellation in the readout) do not turn a rounding-level
difference into an unbounded ratio.  Pass thresholds: 1e-4 for float32 I/O and
2e-2 for bfloat16 I/O with float32 state.
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def metrics(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref.shape}")
    diff = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    floor = rms if rms > 0 else 1.0
    floored = diff / (np.abs(ref) + floor)
    return {
        "floored_max": float(floored.max()) if ref.size else 0.0,
        "normwise": float(diff.max() / max(np.abs(ref).max(), 1e-300)) if ref.size else 0.0,
        "p999_elementwise": float(np.quantile(diff / np.maximum(np.abs(ref), 1e-300), 0.999)) if ref.size else 0.0,
        "rms": rms,
    }
