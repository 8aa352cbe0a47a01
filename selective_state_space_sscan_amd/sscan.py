"""Thin ctypes binding of ``libsscan.so`` (the C ABI in include/sscan.h).

Argument marshalling only: every step of the scan runs in the library's HIP
kernels.  PyTorch supplies device memory (inputs, outputs, the workspace) and the
current stream.  If the library is missing this module raises; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsscan.so")

SSCAN_F32 = 0
SSCAN_BF16 = 1
DSTATE = 16
PROFILE_EVENTS = 5  # step boundaries: start, staged B/C, aggregates, carry, output
PROFILE_STEPS = ("stage_bc", "aggregate", "carry", "output")
BWD_PROFILE_EVENTS = 6  # start, staged B/C, window states, window adjoints, window pass, sums
BWD_PROFILE_STEPS = ("stage_bc", "window_states", "window_adjoints", "window_pass", "param_sums")

_DT_CODE = {torch.float32: SSCAN_F32, torch.bfloat16: SSCAN_BF16}


class SScanError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({strerror(status)})")
        self.status = status


class DirParams(ctypes.Structure):
    _fields_ = [("delta", ctypes.c_void_p), ("delta_bias", ctypes.c_void_p), ("A", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p)]


class ConvParams(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("width", ctypes.c_int),
                ("same", ctypes.c_int), ("silu", ctypes.c_int)]


class DirGrads(ctypes.Structure):
    _fields_ = [("ddelta", ctypes.c_void_p), ("ddelta_bias", ctypes.c_void_p), ("dA", ctypes.c_void_p),
                ("dB", ctypes.c_void_p), ("dC", ctypes.c_void_p), ("dD", ctypes.c_void_p)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads (once) and returns the shared library; raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m selective_state_space_sscan_amd.build`")
    lib = ctypes.CDLL(p)
    V, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    DP = ctypes.POINTER(DirParams)
    lib.sscan_fwd.argtypes = [V, V, V, I, V, V, V, V, V, V, I64, I64, I64, I64, I, V, I, I, V, SZ]
    lib.sscan_fwd.restype = I
    lib.sscan_bidir.argtypes = [V, V, V, DP, DP, I, I64, I64, I64, I64, V, I, I, V, SZ]
    lib.sscan_bidir.restype = I
    lib.sscan_fwd_noalloc.argtypes = lib.sscan_fwd.argtypes[:-2]
    lib.sscan_fwd_noalloc.restype = I
    lib.sscan_fwd_profiled.argtypes = lib.sscan_fwd.argtypes + [V]
    lib.sscan_fwd_profiled.restype = I
    lib.sscan_bidir_profiled.argtypes = lib.sscan_bidir.argtypes + [V]
    lib.sscan_bidir_profiled.restype = I
    lib.sscan_validate_fwd.argtypes = [V, V, V, I, V, V, V, V, V, V, I64, I64, I64, I64, I, I, I, V, SZ]
    lib.sscan_validate_fwd.restype = I
    lib.sscan_validate_bidir.argtypes = [V, V, V, DP, DP, I, I64, I64, I64, I64, I, I, V, SZ]
    lib.sscan_validate_bidir.restype = I
    lib.sscan_fwd_state.argtypes = [V, V, V, I, V, V, V, V, V, V, V, V, I64, I64, I64, I64, I, V, I, I, V, SZ]
    lib.sscan_fwd_state.restype = I
    lib.sscan_validate_fwd_state.argtypes = [V, V, V, I, V, V, V, V, V, V, V, V, I64, I64, I64, I64, I, I, I, V, SZ]
    lib.sscan_validate_fwd_state.restype = I
    lib.sscan_step.argtypes = [V, V, V, V, I, V, V, V, V, V, V, I64, I64, I64, V, I, I]
    lib.sscan_step.restype = I
    lib.sscan_validate_step.argtypes = [V, V, V, V, I, V, V, V, V, V, V, I64, I64, I64, I, I]
    lib.sscan_validate_step.restype = I
    CPP = ctypes.POINTER(ConvParams)
    DGP = ctypes.POINTER(DirGrads)
    lib.sscan_bwd_conv.argtypes = [V, CPP, V, V, I, V, V, V, V, V, V, V, V, DGP, V, V, I64, I64, I64, I64, I, V, I, I,
                                   V, SZ]
    lib.sscan_bwd_conv.restype = I
    lib.sscan_bidir_bwd_conv.argtypes = [V, CPP, V, V, V, V, DP, DP, DGP, DGP, V, V, I, I64, I64, I64, I64, V, I, I, V,
                                         SZ]
    lib.sscan_bidir_bwd_conv.restype = I
    lib.sscan_validate_bwd_conv.argtypes = [V, CPP, V, V, I, V, V, V, V, V, V, V, V, DGP, V, V, I64, I64, I64, I64, I,
                                            I, I, V, SZ]
    lib.sscan_validate_bwd_conv.restype = I
    lib.sscan_bwd_conv_workspace_bytes.argtypes = [I64, I64, I64, I64, I, I]
    lib.sscan_bwd_conv_workspace_bytes.restype = SZ
    lib.sscan_step_conv.argtypes = [V, V, V, CPP, V, V, I, V, V, V, V, V, V, I64, I64, I64, V, I, I]
    lib.sscan_step_conv.restype = I
    lib.sscan_validate_step_conv.argtypes = [V, V, V, CPP, V, V, I, V, V, V, V, V, V, I64, I64, I64, I, I]
    lib.sscan_validate_step_conv.restype = I
    DG = ctypes.POINTER(DirGrads)
    lib.sscan_bwd.argtypes = [V, V, V, I, V, V, V, V, V, V, V, V, DG, I64, I64, I64, I64, I, V, I, I, V, SZ]
    lib.sscan_bwd.restype = I
    lib.sscan_bidir_bwd.argtypes = [V, V, V, V, V, DP, DP, DG, DG, I, I64, I64, I64, I64, V, I, I, V, SZ]
    lib.sscan_bidir_bwd.restype = I
    lib.sscan_validate_bwd.argtypes = [V, V, V, I, V, V, V, V, V, V, V, V, DG, I64, I64, I64, I64, I, I, I, V, SZ]
    lib.sscan_validate_bwd.restype = I
    lib.sscan_validate_bidir_bwd.argtypes = [V, V, V, V, V, DP, DP, DG, DG, I, I64, I64, I64, I64, I, I, V, SZ]
    lib.sscan_validate_bidir_bwd.restype = I
    lib.sscan_bwd_state.argtypes = [V, V, V, I, V, V, V, V, V, V, V, V, V, V, DG, V, I64, I64, I64, I64, I, V, I, I,
                                    V, SZ]
    lib.sscan_bwd_state.restype = I
    lib.sscan_validate_bwd_state.argtypes = [V, V, V, I, V, V, V, V, V, V, V, V, V, V, DG, V, I64, I64, I64, I64, I,
                                             I, I, V, SZ]
    lib.sscan_validate_bwd_state.restype = I
    lib.sscan_bwd_profiled.argtypes = lib.sscan_bwd.argtypes + [V]
    lib.sscan_bwd_profiled.restype = I
    lib.sscan_bidir_bwd_profiled.argtypes = lib.sscan_bidir_bwd.argtypes + [V]
    lib.sscan_bidir_bwd_profiled.restype = I
    lib.sscan_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.sscan_bwd_workspace_bytes.restype = SZ
    CP = ctypes.POINTER(ConvParams)
    lib.sscan_conv1d.argtypes = [V, CP, V, I64, I64, I64, V, I]
    lib.sscan_conv1d.restype = I
    lib.sscan_validate_conv1d.argtypes = [V, CP, V, I64, I64, I64, I]
    lib.sscan_validate_conv1d.restype = I
    lib.sscan_fwd_conv.argtypes = [V, CP, V, V, I, V, V, V, V, V, V, I64, I64, I64, I64, I, V, I, I, V, SZ]
    lib.sscan_fwd_conv.restype = I
    lib.sscan_bidir_conv.argtypes = [V, CP, V, V, DP, DP, I, I64, I64, I64, I64, V, I, I, V, SZ]
    lib.sscan_bidir_conv.restype = I
    lib.sscan_fwd_conv_profiled.argtypes = lib.sscan_fwd_conv.argtypes + [V]
    lib.sscan_fwd_conv_profiled.restype = I
    lib.sscan_bidir_conv_profiled.argtypes = lib.sscan_bidir_conv.argtypes + [V]
    lib.sscan_bidir_conv_profiled.restype = I
    IP = ctypes.POINTER(ctypes.c_int)
    lib.sscan_multi.argtypes = [V, V, V, DP, IP, I, V, I, I64, I64, I64, I64, I64, V, I, I, V, SZ]
    lib.sscan_multi.restype = I
    lib.sscan_validate_multi.argtypes = [V, V, V, DP, IP, I, V, I, I64, I64, I64, I64, I64, I, I, V, SZ]
    lib.sscan_validate_multi.restype = I
    lib.sscan_multi_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, IP, I, I, I]
    lib.sscan_multi_workspace_bytes.restype = SZ
    lib.sscan_multi_bwd.argtypes = [V, V, V, V, V, DP, DG, IP, I, V, I, I64, I64, I64, I64, I64, V, I, I, V, SZ]
    lib.sscan_multi_bwd.restype = I
    lib.sscan_validate_multi_bwd.argtypes = [V, V, V, V, V, DP, DG, IP, I, V, I, I64, I64, I64, I64, I64, I, I, V,
                                             SZ]
    lib.sscan_validate_multi_bwd.restype = I
    lib.sscan_multi_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, IP, I, I, I]
    lib.sscan_multi_bwd_workspace_bytes.restype = SZ
    lib.sscan_spiral_order.argtypes = [I64, I64, V]
    lib.sscan_spiral_order.restype = I
    lib.sscan_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.sscan_workspace_bytes.restype = SZ
    lib.sscan_scan_plan.argtypes = [I64, I64, I64, I64, I, ctypes.POINTER(ctypes.c_int64)]
    lib.sscan_scan_plan.restype = I
    lib.sscan_bwd_plan.argtypes = [I64, I64, I64, I64, I, ctypes.POINTER(ctypes.c_int64)]
    lib.sscan_bwd_plan.restype = I
    lib.sscan_strerror.argtypes = [I]
    lib.sscan_strerror.restype = ctypes.c_char_p
    lib.sscan_version.argtypes = []
    lib.sscan_version.restype = I
    if path is None:
        _lib = lib
    return lib


class HipEvents:
    """Timing events of the HIP runtime the library runs on, for the profiled entry
    points (one set per call in flight): one event per boundary of ``steps``
    (PROFILE_STEPS for the forward calls, BWD_PROFILE_STEPS for the backward)."""

    _hip = None

    def __init__(self, steps=PROFILE_STEPS):
        self.steps = tuple(steps)
        nev = len(self.steps) + 1
        if HipEvents._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already mapped by torch and libsscan
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvents._hip = hip
        self._ev = (ctypes.c_void_p * nev)()
        for i in range(nev):
            h = ctypes.c_void_p()
            if HipEvents._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self._ev[i] = h

    @property
    def handles(self):
        return self._ev

    def step_ms(self):
        """Milliseconds of each step (dict keyed by PROFILE_STEPS); waits for the last event."""
        hip = HipEvents._hip
        hip.hipEventSynchronize(self._ev[len(self.steps)])
        out = {}
        for i, name in enumerate(self.steps):
            ms = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(ms), self._ev[i], self._ev[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = float(ms.value)
        return out

    def total_ms(self) -> float:
        """Milliseconds from the first to the last event (the whole call)."""
        hip = HipEvents._hip
        hip.hipEventSynchronize(self._ev[len(self.steps)])
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), self._ev[0], self._ev[len(self.steps)]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        # through the instance's class: at interpreter exit the module's globals may
        # already be gone when the last events are collected
        hip = getattr(type(self), "_hip", None)
        if hip is not None:
            for h in self._ev:
                if h:
                    hip.hipEventDestroy(h)


def strerror(status: int) -> str:
    return load_library().sscan_strerror(int(status)).decode()


def workspace_bytes(batch: int, dim: int, length: int, dstate: int = DSTATE, bidir: bool = False) -> int:
    return int(load_library().sscan_workspace_bytes(batch, dim, length, dstate, int(bool(bidir))))


def scan_plan(batch: int, dim: int, length: int, dstate: int = DSTATE, bidir: bool = False) -> dict:
    """How a scan of these sizes is split (sscan_scan_plan): segment length, segments
    per row, segments per aggregate run, runs per row."""
    out = (ctypes.c_int64 * 4)()
    st = load_library().sscan_scan_plan(batch, dim, length, dstate, int(bool(bidir)), out)
    if st != 0:
        raise SScanError(st, "sscan_scan_plan")
    return dict(seg_len=out[0], nseg=out[1], run_len=out[2], nrun=out[3])


def bwd_plan(batch: int, dim: int, length: int, dstate: int = DSTATE, bidir: bool = False) -> dict:
    """How a backward call of these sizes is split (sscan_bwd_plan): windows per
    row, blocks per window, channel groups per block, windows per chain run, runs
    per row."""
    out = (ctypes.c_int64 * 5)()
    st = load_library().sscan_bwd_plan(batch, dim, length, dstate, int(bool(bidir)), out)
    if st != 0:
        raise SScanError(st, "sscan_bwd_plan")
    return dict(nwin=out[0], csplit=out[1], gps=out[2], run_len=out[3], nrun=out[4])


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: Optional[torch.Tensor], name: str, device, dtype=None, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check(workspace, "workspace", device)
    return workspace, workspace.numel() * workspace.element_size()


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True, reverse: bool = False,
        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
        events: Optional[HipEvents] = None) -> torch.Tensor:
    """One-direction scan (``sscan_fwd``).  u, delta, z: [batch, dim, len] f32/bf16;
    B, C: [batch, 16, len] f32/bf16; A: [dim, 16] f32; D, delta_bias: [dim] f32.
    Returns the gated output, same dtype as u, enqueued on the current stream.
    With ``events`` the profiled entry point also records the step boundaries."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.fwd needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    _check(u, "u", dev)
    _check(delta, "delta", dev, u.dtype, u.shape)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE, L))
    _check(C, "C", dev, B.dtype, (b, DSTATE, L))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    if out is None:
        out = torch.empty_like(u)
    _check(out, "out", dev, u.dtype, u.shape)
    if u.numel() == 0:
        return out
    ws, ws_bytes = _workspace(workspace_bytes(b, d, L, DSTATE, False), dev, workspace)
    args = [_ptr(u), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(out), b, d, L, DSTATE, int(bool(reverse)), _stream(dev), _DT_CODE[u.dtype], _DT_CODE[B.dtype],
            _ptr(ws), ws_bytes]
    if events is None:
        st = lib.sscan_fwd(*args)
    else:
        if events.steps != PROFILE_STEPS:
            raise ValueError("sscan.fwd needs HipEvents(PROFILE_STEPS)")
        st = lib.sscan_fwd_profiled(*args, ctypes.cast(events.handles, ctypes.c_void_p))
    if st != 0:
        raise SScanError(st, "sscan_fwd")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # SSCAN_NOALLOC_SCRATCH_BYTES


def fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True, reverse: bool = False,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``sscan_fwd_noalloc``: ``fwd`` with the library's fixed scratch array of the
    current device as its workspace (for callers that cannot allocate).  Allocates
    only ``out`` when it is not given."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.fwd_noalloc needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    _check(u, "u", dev)
    _check(delta, "delta", dev, u.dtype, u.shape)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE, L))
    _check(C, "C", dev, B.dtype, (b, DSTATE, L))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    if out is None:
        out = torch.empty_like(u)
    _check(out, "out", dev, u.dtype, u.shape)
    st = lib.sscan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A), _ptr(B), _ptr(C),
                               _ptr(D), _ptr(z), _ptr(out), b, d, L, DSTATE, int(bool(reverse)), _stream(dev),
                               _DT_CODE[u.dtype], _DT_CODE[B.dtype])
    if st != 0:
        raise SScanError(st, "sscan_fwd_noalloc")
    return out


def fwd_state(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0: Optional[torch.Tensor] = None,
              h_last: Optional[torch.Tensor] = None, softplus: bool = True, reverse: bool = False,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """One-direction scan with state I/O (``sscan_fwd_state``).  h0 (optional) is
    the state before the first scanned token, [batch, dim, 16] f32; the state after
    the last scanned token is written to ``h_last`` (allocated if None, may be h0
    itself).  Returns (out, h_last)."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.fwd_state needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    _check(u, "u", dev)
    _check(delta, "delta", dev, u.dtype, u.shape)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE, L))
    _check(C, "C", dev, B.dtype, (b, DSTATE, L))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    _check(h0, "h0", dev, torch.float32, (b, d, DSTATE))
    if h_last is None:
        h_last = torch.empty((b, d, DSTATE), dtype=torch.float32, device=dev)
    _check(h_last, "h_last", dev, torch.float32, (b, d, DSTATE))
    if out is None:
        out = torch.empty_like(u)
    _check(out, "out", dev, u.dtype, u.shape)
    if b * d == 0:
        return out, h_last
    ws, ws_bytes = _workspace(workspace_bytes(b, d, L, DSTATE, False), dev, workspace)
    st = lib.sscan_fwd_state(_ptr(u), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), _ptr(z), _ptr(out), _ptr(h0), _ptr(h_last), b, d, L, DSTATE,
                             int(bool(reverse)), _stream(dev), _DT_CODE[u.dtype], _DT_CODE[B.dtype], _ptr(ws),
                             ws_bytes)
    if st != 0:
        raise SScanError(st, "sscan_fwd_state")
    return out, h_last


def step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token from a stored state (``sscan_step``), updating ``state``
    [batch, dim, 16] f32 in place.  u, delta, z: [batch, dim]; B, C: [batch, 16].
    Returns y [batch, dim] in u's dtype."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.step needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d = u.shape
    _check(state, "state", dev, torch.float32, (b, d, DSTATE))
    _check(u, "u", dev)
    _check(delta, "delta", dev, u.dtype, u.shape)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE))
    _check(C, "C", dev, B.dtype, (b, DSTATE))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    if out is None:
        out = torch.empty_like(u)
    _check(out, "out", dev, u.dtype, u.shape)
    if u.numel() == 0:
        return out
    st = lib.sscan_step(_ptr(state), _ptr(u), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A), _ptr(B),
                        _ptr(C), _ptr(D), _ptr(z), _ptr(out), b, d, DSTATE, _stream(dev), _DT_CODE[u.dtype],
                        _DT_CODE[B.dtype])
    if st != 0:
        raise SScanError(st, "sscan_step")
    return out


def step_conv(state, conv_state, x, conv: dict, delta, A, B, C, D=None, z=None, delta_bias=None,
              softplus: bool = True, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token through the causal convolution and the scan (``sscan_step_conv``):
    ``conv_state`` [batch, dim, width - 1] (x's dtype, may be None for width 1) and
    ``state`` [batch, dim, 16] f32 are updated in place; x, delta, z [batch, dim];
    B, C [batch, 16]; ``conv`` holds weight [dim, width] f32 and optional bias and
    silu.  Returns y [batch, dim] in x's dtype."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("sscan.step_conv needs CUDA (HIP) tensors")
    if x.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("x/delta/z and B/C must be float32 or bfloat16")
    if conv.get("same", False):
        raise ValueError("the decode step needs a causal convolution")
    b, d = x.shape
    cp = _conv_params(dict(conv, same=False), d, dev)
    _check(state, "state", dev, torch.float32, (b, d, DSTATE))
    _check(conv_state, "conv_state", dev, x.dtype, (b, d, cp.width - 1))
    _check(x, "x", dev)
    _check(delta, "delta", dev, x.dtype, x.shape)
    _check(z, "z", dev, x.dtype, x.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE))
    _check(C, "C", dev, B.dtype, (b, DSTATE))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", dev, x.dtype, x.shape)
    if x.numel() == 0:
        return out
    st = lib.sscan_step_conv(_ptr(state), _ptr(conv_state) if conv_state is not None and conv_state.numel() else None,
                             _ptr(x), ctypes.byref(cp), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A),
                             _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(out), b, d, DSTATE, _stream(dev),
                             _DT_CODE[x.dtype], _DT_CODE[B.dtype])
    if st != 0:
        raise SScanError(st, "sscan_step_conv")
    return out


def _dir(p: dict, name: str, dev, u, bdtype):
    b, d, L = u.shape
    _check(p["delta"], f"{name}.delta", dev, u.dtype, u.shape)
    _check(p["A"], f"{name}.A", dev, torch.float32, (d, DSTATE))
    _check(p["B"], f"{name}.B", dev, bdtype, (b, DSTATE, L))
    _check(p["C"], f"{name}.C", dev, bdtype, (b, DSTATE, L))
    _check(p.get("D"), f"{name}.D", dev, torch.float32, (d,))
    _check(p.get("delta_bias"), f"{name}.delta_bias", dev, torch.float32, (d,))
    return DirParams(p["delta"].data_ptr(), p["delta_bias"].data_ptr() if p.get("delta_bias") is not None else None,
                     p["A"].data_ptr(), p["B"].data_ptr(), p["C"].data_ptr(),
                     p["D"].data_ptr() if p.get("D") is not None else None)


def bidir(u, z, fwd: dict, rev: dict, softplus: bool = True, out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None, events: Optional[HipEvents] = None) -> torch.Tensor:
    """Bidirectional scan (``sscan_bidir``): ``fwd`` and ``rev`` are dicts with
    delta, A, B, C and optional D, delta_bias.  Returns (y_fwd + y_rev) * silu(z)."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.bidir needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or fwd["B"].dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    _check(u, "u", dev)
    _check(z, "z", dev, u.dtype, u.shape)
    pf = _dir(fwd, "fwd", dev, u, fwd["B"].dtype)
    pr = _dir(rev, "rev", dev, u, fwd["B"].dtype)
    if out is None:
        out = torch.empty_like(u)
    _check(out, "out", dev, u.dtype, u.shape)
    if u.numel() == 0:
        return out
    ws, ws_bytes = _workspace(workspace_bytes(b, d, L, DSTATE, True), dev, workspace)
    args = [_ptr(u), _ptr(z), _ptr(out), ctypes.byref(pf), ctypes.byref(pr), int(bool(softplus)), b, d, L, DSTATE,
            _stream(dev), _DT_CODE[u.dtype], _DT_CODE[fwd["B"].dtype], _ptr(ws), ws_bytes]
    if events is None:
        st = lib.sscan_bidir(*args)
    else:
        if events.steps != PROFILE_STEPS:
            raise ValueError("sscan.bidir needs HipEvents(PROFILE_STEPS)")
        st = lib.sscan_bidir_profiled(*args, ctypes.cast(events.handles, ctypes.c_void_p))
    if st != 0:
        raise SScanError(st, "sscan_bidir")
    return out


def _conv_params(conv: dict, dim: int, dev) -> ConvParams:
    w = conv["weight"]
    _check(w, "conv weight", dev, torch.float32)
    if w.dim() != 2 or w.shape[0] != dim:
        raise ValueError(f"conv weight must be [dim={dim}, width]")
    _check(conv.get("bias"), "conv bias", dev, torch.float32, (dim,))
    b = conv.get("bias")
    return ConvParams(w.data_ptr(), b.data_ptr() if b is not None else None, int(w.shape[1]),
                      int(bool(conv.get("same", False))), int(bool(conv.get("silu", False))))


def conv1d(x, weight, bias=None, same: bool = False, silu: bool = False,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Depthwise convolution of each channel (``sscan_conv1d``): x [batch, dim, len]
    f32/bf16, weight [dim, width] f32 (causal, or centred when ``same``), optional
    bias [dim] f32, optional silu."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("sscan.conv1d needs CUDA (HIP) tensors")
    if x.dtype not in _DT_CODE:
        raise TypeError("x must be float32 or bfloat16")
    b, d, L = x.shape
    _check(x, "x", dev)
    cp = _conv_params(dict(weight=weight, bias=bias, same=same, silu=silu), d, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", dev, x.dtype, x.shape)
    st = lib.sscan_conv1d(_ptr(x), ctypes.byref(cp), _ptr(out), b, d, L, _stream(dev), _DT_CODE[x.dtype])
    if st != 0:
        raise SScanError(st, "sscan_conv1d")
    return out


def _fwd_events(events: Optional[HipEvents]):
    if events is None:
        return None
    if events.steps != PROFILE_STEPS:
        raise ValueError("the forward calls need HipEvents(PROFILE_STEPS)")
    return ctypes.cast(events.handles, ctypes.c_void_p)


def fwd_conv(x, conv: dict, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
             reverse: bool = False, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, events: Optional[HipEvents] = None) -> torch.Tensor:
    """``sscan_fwd_conv``: the scan of u = conv(x), the convolution computed inside
    the scan kernels.  ``conv`` holds weight [dim, width] f32 and optional bias,
    same, silu."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("sscan.fwd_conv needs CUDA (HIP) tensors")
    if x.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("x/delta/z and B/C must be float32 or bfloat16")
    b, d, L = x.shape
    _check(x, "x", dev)
    _check(delta, "delta", dev, x.dtype, x.shape)
    _check(z, "z", dev, x.dtype, x.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE, L))
    _check(C, "C", dev, B.dtype, (b, DSTATE, L))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    cp = _conv_params(conv, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", dev, x.dtype, x.shape)
    if x.numel() == 0:
        return out
    ws, ws_bytes = _workspace(workspace_bytes(b, d, L, DSTATE, False), dev, workspace)
    args = [_ptr(x), ctypes.byref(cp), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(out), b, d, L, DSTATE, int(bool(reverse)), _stream(dev), _DT_CODE[x.dtype],
            _DT_CODE[B.dtype], _ptr(ws), ws_bytes]
    ev = _fwd_events(events)
    st = lib.sscan_fwd_conv(*args) if ev is None else lib.sscan_fwd_conv_profiled(*args, ev)
    if st != 0:
        raise SScanError(st, "sscan_fwd_conv")
    return out


def bidir_conv(x, conv: dict, z, fwd: dict, rev: dict, softplus: bool = True, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, events: Optional[HipEvents] = None) -> torch.Tensor:
    """``sscan_bidir_conv``: both directions over u = conv(x), summed, gated once."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("sscan.bidir_conv needs CUDA (HIP) tensors")
    if x.dtype not in _DT_CODE or fwd["B"].dtype not in _DT_CODE:
        raise TypeError("x/delta/z and B/C must be float32 or bfloat16")
    b, d, L = x.shape
    _check(x, "x", dev)
    _check(z, "z", dev, x.dtype, x.shape)
    pf = _dir(fwd, "fwd", dev, x, fwd["B"].dtype)
    pr = _dir(rev, "rev", dev, x, fwd["B"].dtype)
    cp = _conv_params(conv, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", dev, x.dtype, x.shape)
    if x.numel() == 0:
        return out
    ws, ws_bytes = _workspace(workspace_bytes(b, d, L, DSTATE, True), dev, workspace)
    args = [_ptr(x), ctypes.byref(cp), _ptr(z), _ptr(out), ctypes.byref(pf), ctypes.byref(pr), int(bool(softplus)), b,
            d, L, DSTATE, _stream(dev), _DT_CODE[x.dtype], _DT_CODE[fwd["B"].dtype], _ptr(ws), ws_bytes]
    ev = _fwd_events(events)
    st = lib.sscan_bidir_conv(*args) if ev is None else lib.sscan_bidir_conv_profiled(*args, ev)
    if st != 0:
        raise SScanError(st, "sscan_bidir_conv")
    return out


ORDER_ROW, ORDER_ROW_REV, ORDER_COL, ORDER_COL_REV, ORDER_INDEX, ORDER_INDEX_REV = range(6)


def spiral_order(height: int, width: int) -> torch.Tensor:
    """The centre-out clockwise spiral over a [height, width] map (``sscan_spiral_order``,
    host code): int32 CPU tensor of row-major token indices."""
    out = torch.empty(height * width, dtype=torch.int32)
    st = load_library().sscan_spiral_order(height, width, ctypes.c_void_p(out.data_ptr()) if out.numel() else None)
    if st != 0:
        raise SScanError(st, "sscan_spiral_order")
    return out


def multi_workspace_bytes(batch, dim, height, width, kinds, io_dtype=torch.float32, bc_dtype=torch.float32) -> int:
    k = (ctypes.c_int * len(kinds))(*kinds)
    return int(load_library().sscan_multi_workspace_bytes(batch, dim, height, width, DSTATE, k, len(kinds),
                                                          _DT_CODE[io_dtype], _DT_CODE[bc_dtype]))


def multi(u, z, dirs, kinds, height: int, width: int, index: Optional[torch.Tensor] = None, softplus: bool = True,
          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``sscan_multi``: the map [height, width] (flattened row-major in u's last
    axis) scanned along the orders ``kinds`` (ORDER_*), one parameter dict per
    direction (delta, A, B, C, optional D, delta_bias, all in token layout); the
    directions' outputs are summed and gated once.  ``index`` (device int32
    permutation) is needed by the index orders."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.multi needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or dirs[0]["B"].dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    if L != height * width:
        raise ValueError("u's last axis must be height * width")
    if len(dirs) != len(kinds):
        raise ValueError("one parameter dict per order")
    _check(u, "u", dev)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(index, "index", dev, torch.int32, (L,))
    bdt = dirs[0]["B"].dtype
    ps = [_dir(p, f"dirs[{k}]", dev, u, bdt) for k, p in enumerate(dirs)]
    arr = (DirParams * len(ps))(*ps)
    kk = (ctypes.c_int * len(kinds))(*kinds)
    if out is None:
        out = torch.empty_like(u)
    _check(out, "out", dev, u.dtype, u.shape)
    if u.numel() == 0:
        return out
    nbytes = multi_workspace_bytes(b, d, height, width, kinds, u.dtype, bdt)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", dev)
    st = lib.sscan_multi(_ptr(u), _ptr(z), _ptr(out), arr, kk, len(kinds), _ptr(index), int(bool(softplus)), b, d,
                         height, width, DSTATE, _stream(dev), _DT_CODE[u.dtype], _DT_CODE[bdt], _ptr(workspace),
                         workspace.numel())
    if st != 0:
        raise SScanError(st, "sscan_multi")
    return out


def multi_bwd_workspace_bytes(batch, dim, height, width, kinds, io_dtype=torch.float32,
                              bc_dtype=torch.float32) -> int:
    k = (ctypes.c_int * len(kinds))(*kinds)
    return int(load_library().sscan_multi_bwd_workspace_bytes(batch, dim, height, width, DSTATE, k, len(kinds),
                                                              _DT_CODE[io_dtype], _DT_CODE[bc_dtype]))


def multi_bwd(u, z, dout, dirs, kinds, height: int, width: int, index: Optional[torch.Tensor] = None,
              softplus: bool = True, workspace: Optional[torch.Tensor] = None) -> dict:
    """Backward pass of ``multi`` (``sscan_multi_bwd``): gradients of
    sum(dout * out).  Returns {"du", "dz" (None without z), "dirs": [one dict per
    direction with ddelta, ddelta_bias, dA, dB, dC, dD as in ``bwd``]}."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.multi_bwd needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or dirs[0]["B"].dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    if L != height * width:
        raise ValueError("u's last axis must be height * width")
    if len(dirs) != len(kinds):
        raise ValueError("one parameter dict per order")
    _check(u, "u", dev)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(dout, "dout", dev, u.dtype, u.shape)
    _check(index, "index", dev, torch.int32, (L,))
    bdt = dirs[0]["B"].dtype
    ps = [_dir(p, f"dirs[{k}]", dev, u, bdt) for k, p in enumerate(dirs)]
    gs = [_grads_for(p, u) for p in dirs]
    arr = (DirParams * len(ps))(*ps)
    garr = (DirGrads * len(gs))(*[g[1] for g in gs])
    kk = (ctypes.c_int * len(kinds))(*kinds)
    du = torch.empty_like(u)
    dz = torch.empty_like(u) if z is not None else None
    nbytes = multi_bwd_workspace_bytes(b, d, height, width, kinds, u.dtype, bdt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", dev)
    st = lib.sscan_multi_bwd(_ptr(u), _ptr(z), _ptr(dout), _ptr(du), _ptr(dz), arr, garr, kk, len(kinds), _ptr(index),
                             int(bool(softplus)), b, d, height, width, DSTATE, _stream(dev), _DT_CODE[u.dtype],
                             _DT_CODE[bdt], _ptr(workspace), workspace.numel())
    if st != 0:
        raise SScanError(st, "sscan_multi_bwd")
    return {"du": du, "dz": dz, "dirs": [g[0] for g in gs]}


def bwd_workspace_bytes(batch: int, dim: int, length: int, dstate: int = DSTATE, bidir: bool = False) -> int:
    return int(load_library().sscan_bwd_workspace_bytes(batch, dim, length, dstate, int(bool(bidir))))


def _grads_for(p: dict, u):
    """Output tensors for one direction's gradients (shapes and dtypes of its inputs)."""
    d = u.shape[1]
    dev = u.device
    g = {"ddelta": torch.empty_like(p["delta"]), "dA": torch.empty_like(p["A"]),
         "dB": torch.empty_like(p["B"]), "dC": torch.empty_like(p["C"]),
         "ddelta_bias": torch.empty(d, dtype=torch.float32, device=dev) if p.get("delta_bias") is not None else None,
         "dD": torch.empty(d, dtype=torch.float32, device=dev) if p.get("D") is not None else None}
    st = DirGrads(g["ddelta"].data_ptr(), g["ddelta_bias"].data_ptr() if g["ddelta_bias"] is not None else None,
                  g["dA"].data_ptr(), g["dB"].data_ptr(), g["dC"].data_ptr(),
                  g["dD"].data_ptr() if g["dD"] is not None else None)
    return g, st


def _bwd_events(events: Optional[HipEvents]):
    if events is None:
        return None
    if events.steps != BWD_PROFILE_STEPS:
        raise ValueError("the backward calls need HipEvents(BWD_PROFILE_STEPS)")
    return ctypes.cast(events.handles, ctypes.c_void_p)


def bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None, softplus: bool = True, reverse: bool = False,
        workspace: Optional[torch.Tensor] = None, events: Optional[HipEvents] = None) -> dict:
    """Backward pass of ``fwd`` (``sscan_bwd``): gradients of sum(dout * out).
    Returns a dict with du, dz (None without z), ddelta, ddelta_bias, dA, dB, dC, dD
    (None for an absent optional input), in the dtypes of the matching inputs."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.bwd needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    _check(u, "u", dev)
    _check(delta, "delta", dev, u.dtype, u.shape)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(dout, "dout", dev, u.dtype, u.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE, L))
    _check(C, "C", dev, B.dtype, (b, DSTATE, L))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    p = dict(delta=delta, A=A, B=B, C=C, D=D, delta_bias=delta_bias)
    g, gst = _grads_for(p, u)
    du = torch.empty_like(u)
    dz = torch.empty_like(u) if z is not None else None
    ws, ws_bytes = _workspace(bwd_workspace_bytes(b, d, L, DSTATE, False), dev, workspace)
    args = [_ptr(u), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(z), _ptr(dout), _ptr(du), _ptr(dz), ctypes.byref(gst), b, d, L, DSTATE, int(bool(reverse)),
            _stream(dev), _DT_CODE[u.dtype], _DT_CODE[B.dtype], _ptr(ws), ws_bytes]
    ev = _bwd_events(events)
    st = lib.sscan_bwd(*args) if ev is None else lib.sscan_bwd_profiled(*args, ev)
    if st != 0:
        raise SScanError(st, "sscan_bwd")
    return dict(g, du=du, dz=dz)


def bwd_state(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None, h0=None, dh_last=None,
              softplus: bool = True, reverse: bool = False, workspace: Optional[torch.Tensor] = None) -> dict:
    """Backward pass of ``fwd_state`` (``sscan_bwd_state``): the gradients of
    sum(dout * out) + sum(dh_last * h_last) given the forward's entry state ``h0``;
    returns ``bwd``'s dict plus "dh0" [batch, dim, 16] f32."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.bwd_state needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    _check(u, "u", dev)
    _check(delta, "delta", dev, u.dtype, u.shape)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(dout, "dout", dev, u.dtype, u.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE, L))
    _check(C, "C", dev, B.dtype, (b, DSTATE, L))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    _check(h0, "h0", dev, torch.float32, (b, d, DSTATE))
    _check(dh_last, "dh_last", dev, torch.float32, (b, d, DSTATE))
    g, gst = _grads_for(dict(delta=delta, A=A, B=B, C=C, D=D, delta_bias=delta_bias), u)
    du = torch.empty_like(u)
    dz = torch.empty_like(u) if z is not None else None
    dh0 = torch.empty((b, d, DSTATE), dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(bwd_workspace_bytes(b, d, L, DSTATE, False), dev, workspace)
    st = lib.sscan_bwd_state(_ptr(u), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), _ptr(z), _ptr(dout), _ptr(h0), _ptr(dh_last), _ptr(du), _ptr(dz),
                             ctypes.byref(gst), _ptr(dh0), b, d, L, DSTATE, int(bool(reverse)), _stream(dev),
                             _DT_CODE[u.dtype], _DT_CODE[B.dtype], _ptr(ws), ws_bytes)
    if st != 0:
        raise SScanError(st, "sscan_bwd_state")
    return dict(g, du=du, dz=dz, dh0=dh0)


def bidir_bwd(u, z, dout, fwd: dict, rev: dict, softplus: bool = True,
              workspace: Optional[torch.Tensor] = None, events: Optional[HipEvents] = None) -> dict:
    """Backward pass of ``bidir`` (``sscan_bidir_bwd``).  Returns {"du", "dz",
    "fwd": {...}, "rev": {...}} with each direction's gradients as in ``bwd``."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("sscan.bidir_bwd needs CUDA (HIP) tensors")
    if u.dtype not in _DT_CODE or fwd["B"].dtype not in _DT_CODE:
        raise TypeError("u/delta/z and B/C must be float32 or bfloat16")
    b, d, L = u.shape
    _check(u, "u", dev)
    _check(z, "z", dev, u.dtype, u.shape)
    _check(dout, "dout", dev, u.dtype, u.shape)
    pf = _dir(fwd, "fwd", dev, u, fwd["B"].dtype)
    pr = _dir(rev, "rev", dev, u, fwd["B"].dtype)
    gf, gfs = _grads_for(fwd, u)
    gr, grs = _grads_for(rev, u)
    du = torch.empty_like(u)
    dz = torch.empty_like(u) if z is not None else None
    ws, ws_bytes = _workspace(bwd_workspace_bytes(b, d, L, DSTATE, True), dev, workspace)
    args = [_ptr(u), _ptr(z), _ptr(dout), _ptr(du), _ptr(dz), ctypes.byref(pf), ctypes.byref(pr),
            ctypes.byref(gfs), ctypes.byref(grs), int(bool(softplus)), b, d, L, DSTATE, _stream(dev),
            _DT_CODE[u.dtype], _DT_CODE[fwd["B"].dtype], _ptr(ws), ws_bytes]
    ev = _bwd_events(events)
    st = lib.sscan_bidir_bwd(*args) if ev is None else lib.sscan_bidir_bwd_profiled(*args, ev)
    if st != 0:
        raise SScanError(st, "sscan_bidir_bwd")
    return {"du": du, "dz": dz, "fwd": gf, "rev": gr}


def bwd_conv_workspace_bytes(batch: int, dim: int, length: int, dstate: int = DSTATE, bidir: bool = False,
                             io_dtype=torch.float32) -> int:
    return int(load_library().sscan_bwd_conv_workspace_bytes(batch, dim, length, dstate, int(bool(bidir)),
                                                             _DT_CODE[io_dtype]))


def _conv_grads(conv: dict, dim: int, dev):
    dw = torch.empty((dim, conv["weight"].shape[1]), dtype=torch.float32, device=dev)
    db = torch.empty(dim, dtype=torch.float32, device=dev) if conv.get("bias") is not None else None
    return dw, db


def bwd_conv(x, conv: dict, delta, A, B, C, dout, D=None, z=None, delta_bias=None, softplus: bool = True,
             reverse: bool = False, workspace: Optional[torch.Tensor] = None) -> dict:
    """Backward of ``fwd_conv`` (``sscan_bwd_conv``): the gradients of ``bwd`` with
    dx in place of du, plus dconv_w [dim, width] and dconv_b [dim] (None without a
    convolution bias)."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("sscan.bwd_conv needs CUDA (HIP) tensors")
    if x.dtype not in _DT_CODE or B.dtype not in _DT_CODE:
        raise TypeError("x/delta/z and B/C must be float32 or bfloat16")
    b, d, L = x.shape
    _check(x, "x", dev)
    _check(delta, "delta", dev, x.dtype, x.shape)
    _check(z, "z", dev, x.dtype, x.shape)
    _check(dout, "dout", dev, x.dtype, x.shape)
    _check(A, "A", dev, torch.float32, (d, DSTATE))
    _check(B, "B", dev, None, (b, DSTATE, L))
    _check(C, "C", dev, B.dtype, (b, DSTATE, L))
    _check(D, "D", dev, torch.float32, (d,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (d,))
    cp = _conv_params(conv, d, dev)
    g, gst = _grads_for(dict(delta=delta, A=A, B=B, C=C, D=D, delta_bias=delta_bias), x)
    dx = torch.empty_like(x)
    dz = torch.empty_like(x) if z is not None else None
    dw, db = _conv_grads(conv, d, dev)
    nbytes = bwd_conv_workspace_bytes(b, d, L, DSTATE, False, x.dtype)
    ws, ws_bytes = _workspace(nbytes, dev, workspace)
    st = lib.sscan_bwd_conv(_ptr(x), ctypes.byref(cp), _ptr(delta), _ptr(delta_bias), int(bool(softplus)), _ptr(A),
                            _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dout), _ptr(dx), _ptr(dz), ctypes.byref(gst),
                            _ptr(dw), _ptr(db), b, d, L, DSTATE, int(bool(reverse)), _stream(dev), _DT_CODE[x.dtype],
                            _DT_CODE[B.dtype], _ptr(ws), ws_bytes)
    if st != 0:
        raise SScanError(st, "sscan_bwd_conv")
    return dict(g, dx=dx, dz=dz, dconv_w=dw, dconv_b=db)


def bidir_bwd_conv(x, conv: dict, z, dout, fwd: dict, rev: dict, softplus: bool = True,
                   workspace: Optional[torch.Tensor] = None) -> dict:
    """Backward of ``bidir_conv`` (``sscan_bidir_bwd_conv``): {"dx", "dz", "dconv_w",
    "dconv_b", "fwd": {...}, "rev": {...}}."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("sscan.bidir_bwd_conv needs CUDA (HIP) tensors")
    if x.dtype not in _DT_CODE or fwd["B"].dtype not in _DT_CODE:
        raise TypeError("x/delta/z and B/C must be float32 or bfloat16")
    b, d, L = x.shape
    _check(x, "x", dev)
    _check(z, "z", dev, x.dtype, x.shape)
    _check(dout, "dout", dev, x.dtype, x.shape)
    pf = _dir(fwd, "fwd", dev, x, fwd["B"].dtype)
    pr = _dir(rev, "rev", dev, x, fwd["B"].dtype)
    cp = _conv_params(conv, d, dev)
    gf, gfs = _grads_for(fwd, x)
    gr, grs = _grads_for(rev, x)
    dx = torch.empty_like(x)
    dz = torch.empty_like(x) if z is not None else None
    dw, db = _conv_grads(conv, d, dev)
    nbytes = bwd_conv_workspace_bytes(b, d, L, DSTATE, True, x.dtype)
    ws, ws_bytes = _workspace(nbytes, dev, workspace)
    st = lib.sscan_bidir_bwd_conv(_ptr(x), ctypes.byref(cp), _ptr(z), _ptr(dout), _ptr(dx), _ptr(dz),
                                  ctypes.byref(pf), ctypes.byref(pr), ctypes.byref(gfs), ctypes.byref(grs), _ptr(dw),
                                  _ptr(db), int(bool(softplus)), b, d, L, DSTATE, _stream(dev), _DT_CODE[x.dtype],
                                  _DT_CODE[fwd["B"].dtype], _ptr(ws), ws_bytes)
    if st != 0:
        raise SScanError(st, "sscan_bidir_bwd_conv")
    return {"dx": dx, "dz": dz, "dconv_w": dw, "dconv_b": db, "fwd": gf, "rev": gr}


def run_inputs(x, softplus: bool = True, out=None, workspace=None, events: Optional[HipEvents] = None) -> torch.Tensor:
    """Runs the scan on a ``ScanInputs`` already on the device (one or two directions)."""
    if len(x.dirs) == 1:
        p = x.dirs[0]
        return fwd(x.u, x.delta, p.A, p.B, p.C, p.D, x.z, p.delta_bias, softplus=softplus, out=out,
                   workspace=workspace, events=events)
    f, r = x.dirs
    mk = lambda p: dict(delta=x.delta, delta_bias=p.delta_bias, A=p.A, B=p.B, C=p.C, D=p.D)
    return bidir(x.u, x.z, mk(f), mk(r), softplus=softplus, out=out, workspace=workspace, events=events)


# ---- autograd ---------------------------------------------------------------------
# torch.autograd.Function wrappers: the forward call, and in backward the matching
# backward entry point (the forward states are recomputed there, nothing beyond the
# inputs is kept).  Argument marshalling only, like the functions above.

class _ScanFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, delta, A, B, C, D, z, delta_bias, softplus, reverse):
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias)
        ctx.softplus, ctx.reverse = softplus, reverse
        return fwd(u, delta, A, B, C, D, z, delta_bias, softplus=softplus, reverse=reverse)

    @staticmethod
    def backward(ctx, dout):
        u, delta, A, B, C, D, z, delta_bias = ctx.saved_tensors
        g = bwd(u, delta, A, B, C, dout.contiguous(), D=D, z=z, delta_bias=delta_bias, softplus=ctx.softplus,
                reverse=ctx.reverse)
        return (g["du"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"], g["ddelta_bias"], None, None)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                   reverse: bool = False) -> torch.Tensor:
    """``fwd`` with gradients: differentiable in every tensor argument (``sscan_bwd``
    in the backward pass)."""
    return _ScanFn.apply(u, delta, A, B, C, D, z, delta_bias, softplus, reverse)


class _BidirFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, z, d_f, A_f, B_f, C_f, D_f, bias_f, d_r, A_r, B_r, C_r, D_r, bias_r, softplus):
        ctx.save_for_backward(u, z, d_f, A_f, B_f, C_f, D_f, bias_f, d_r, A_r, B_r, C_r, D_r, bias_r)
        ctx.softplus = softplus
        pf = dict(delta=d_f, A=A_f, B=B_f, C=C_f, D=D_f, delta_bias=bias_f)
        pr = dict(delta=d_r, A=A_r, B=B_r, C=C_r, D=D_r, delta_bias=bias_r)
        return bidir(u, z, pf, pr, softplus=softplus)

    @staticmethod
    def backward(ctx, dout):
        u, z, d_f, A_f, B_f, C_f, D_f, bias_f, d_r, A_r, B_r, C_r, D_r, bias_r = ctx.saved_tensors
        pf = dict(delta=d_f, A=A_f, B=B_f, C=C_f, D=D_f, delta_bias=bias_f)
        pr = dict(delta=d_r, A=A_r, B=B_r, C=C_r, D=D_r, delta_bias=bias_r)
        g = bidir_bwd(u, z, dout.contiguous(), pf, pr, softplus=ctx.softplus)
        gf, gr = g["fwd"], g["rev"]
        # a delta tensor shared by the two directions appears twice in the inputs, and
        # autograd adds the two gradients it receives for it
        return (g["du"], g["dz"],
                gf["ddelta"], gf["dA"], gf["dB"], gf["dC"], gf["dD"], gf["ddelta_bias"],
                gr["ddelta"], gr["dA"], gr["dB"], gr["dC"], gr["dD"], gr["ddelta_bias"], None)


def selective_scan_bidir(u, z, fwd_params: dict, rev_params: dict, softplus: bool = True) -> torch.Tensor:
    """``bidir`` with gradients (``sscan_bidir_bwd`` in the backward pass); each
    parameter dict holds delta, A, B, C and optional D, delta_bias."""
    f, r = fwd_params, rev_params
    return _BidirFn.apply(u, z, f["delta"], f["A"], f["B"], f["C"], f.get("D"), f.get("delta_bias"),
                          r["delta"], r["A"], r["B"], r["C"], r.get("D"), r.get("delta_bias"), softplus)
