"""Seeded synthetic inputs for the selective scan (S6).

This module only draws random numbers and casts them to storage dtypes; it holds
none of the scan's arithmetic.  Both the fp64 oracle (test infrastructure) and the
HIP path are fed from here, so they always see the same values.

Recipe (one numpy PCG64 generator per call, ``numpy.random.default_rng(seed)``;
draw order is fixed as listed):

* ``u``      ~ N(0, 1), shape [batch, dim, len], drawn in float32;
* ``delta``  = 0.5 * N(0, 1), shape [batch, dim, len], drawn in float32 (raw, before
  bias and softplus; shared by both directions of a bidirectional scan);
* ``z``      ~ N(0, 1), shape [batch, dim, len], drawn in float32;
* then, per direction (forward first, then reverse):
  - ``A``: with ``a_init="s4d"`` (the workloads' recipe) ``A[d, n] = -(n + 1)``
    (S4D-real initialisation, no draw); with ``a_init="random"`` (the default of
    ``make_inputs``) ``A[d, n] = -exp(a_log[d, n])`` with ``a_log ~ U(-1, 1.5)``
    drawn per (channel, state), the learned parameterisation A = -exp(A_log) of the
    Hand-written simplified Mamba2 page (sections 4.2 and 4.4), so every channel
    and state has its own decay; float32;
  - ``v_d`` log-uniform in ``dt_range``; ``delta_bias_d = log(expm1(v_d))``
    (the value whose softplus is ``v_d``), float64 then float32;
  - ``D_d`` ~ N(0, 1), float64 then float32;
  - ``B``, ``C`` ~ N(0, 1), shape [batch, dstate, len], float64.

Per-token tensors are cast to the I/O dtype (``f32`` or ``bf16``) and B/C to their
own dtype by torch (round to nearest even).  The oracle reads back exactly the cast
values, widened to float64, so input quantisation is never counted as error.

The workload shapes mirror the pages: Vision Mamba's 14x14 patches plus a cls
token (197 tokens, Reproducing Vision Mamba page, section 3.1), the Mamba-YOLO
stage-1 128x128 row-major map (Mamba in the YOLO26 backbone page, section 2.2) and
sequences of hundreds of thousands of tokens (Hand-written simplified Mamba2 page,
opening).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

DSTATE = 16

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    """One workload: shapes, number of directions and storage dtypes."""

    name: str
    batch: int
    dim: int
    len: int
    bidir: bool
    io_dtype: str  # dtype of u, delta, z and the output y
    bc_dtype: str  # dtype of B and C
    dt_range: Tuple[float, float] = (1e-3, 1e-1)
    dstate: int = DSTATE

    @property
    def elems(self) -> int:
        return self.batch * self.dim * self.len

    @property
    def ndir(self) -> int:
        return 2 if self.bidir else 1


CONFIGS: List[ScanConfig] = [
    ScanConfig("tiny-fwd", 2, 64, 32, False, "f32", "f32"),
    ScanConfig("vim-tiny-bidir", 64, 384, 197, True, "f32", "f32"),
    ScanConfig("vim-small-bidir", 128, 768, 197, True, "bf16", "bf16"),
    ScanConfig("yolo-stage1-rowbidir", 8, 192, 16384, True, "bf16", "bf16"),
    ScanConfig("long-seq-fwd", 1, 1536, 262144, False, "bf16", "f32", (1e-4, 1e-2)),
]


def config_seed(cfg_index: int, k: int = 0) -> int:
    """Seed of the k-th draw of config ``cfg_index``."""
    return 1000 * cfg_index + k


@dataclasses.dataclass
class DirParams:
    """Per-direction parameters (torch CPU tensors in storage dtype)."""

    delta_bias: torch.Tensor  # [dim] f32
    A: torch.Tensor  # [dim, dstate] f32
    B: torch.Tensor  # [batch, dstate, len] bc dtype
    C: torch.Tensor  # [batch, dstate, len] bc dtype
    D: torch.Tensor  # [dim] f32


@dataclasses.dataclass
class ScanInputs:
    """All inputs of one scan call (torch CPU tensors in storage dtype)."""

    u: torch.Tensor  # [batch, dim, len]
    delta: torch.Tensor  # [batch, dim, len]
    z: torch.Tensor  # [batch, dim, len]
    dirs: List[DirParams]
    io_dtype: str
    bc_dtype: str

    @property
    def shape(self) -> Tuple[int, int, int]:
        b, d, l = self.u.shape
        return b, d, l

    @property
    def dstate(self) -> int:
        return self.dirs[0].A.shape[1]

    def tensors(self) -> List[torch.Tensor]:
        """Every distinct input tensor (each direction's parameters included)."""
        ts = [self.u, self.delta, self.z]
        for p in self.dirs:
            ts += [p.delta_bias, p.A, p.B, p.C, p.D]
        return ts

    def clone(self) -> "ScanInputs":
        """The same values in new storage (on the same device)."""
        return ScanInputs(
            self.u.clone(), self.delta.clone(), self.z.clone(),
            [DirParams(p.delta_bias.clone(), p.A.clone(), p.B.clone(), p.C.clone(), p.D.clone()) for p in self.dirs],
            self.io_dtype, self.bc_dtype)

    def to(self, device) -> "ScanInputs":
        mv = lambda t: t.to(device, non_blocking=False).contiguous()
        return ScanInputs(
            mv(self.u), mv(self.delta), mv(self.z),
            [DirParams(mv(p.delta_bias), mv(p.A), mv(p.B), mv(p.C), mv(p.D)) for p in self.dirs],
            self.io_dtype, self.bc_dtype)


def _cast(arr: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr)).to(_TORCH_DTYPES[dtype]).contiguous()


def make_inputs(batch: int, dim: int, length: int, *, dstate: int = DSTATE, bidir: bool = False,
                io_dtype: str = "f32", bc_dtype: str = "f32", seed: int = 0,
                dt_range: Tuple[float, float] = (1e-3, 1e-1), a_init: str = "random") -> ScanInputs:
    """Draw one seeded set of inputs (see the module docstring for the recipe)."""
    if a_init not in ("s4d", "random"):
        raise ValueError(f"a_init must be 's4d' or 'random', not {a_init!r}")
    rng = np.random.default_rng(seed)
    shp = (batch, dim, length)
    u = rng.standard_normal(shp, dtype=np.float32)
    delta = rng.standard_normal(shp, dtype=np.float32)
    delta *= np.float32(0.5)
    z = rng.standard_normal(shp, dtype=np.float32)
    dirs = []
    lo, hi = np.log(dt_range[0]), np.log(dt_range[1])
    for _ in range(2 if bidir else 1):
        if a_init == "s4d":
            A = -np.broadcast_to(np.arange(1, dstate + 1, dtype=np.float64), (dim, dstate))
        else:
            A = -np.exp(rng.uniform(-1.0, 1.5, size=(dim, dstate)))
        v = np.exp(rng.uniform(lo, hi, size=dim))
        bias = np.log(np.expm1(v))
        D = rng.standard_normal(dim)
        B = rng.standard_normal((batch, dstate, length))
        C = rng.standard_normal((batch, dstate, length))
        dirs.append(DirParams(_cast(bias, "f32"), _cast(A, "f32"), _cast(B, bc_dtype),
                              _cast(C, bc_dtype), _cast(D, "f32")))
    return ScanInputs(_cast(u, io_dtype), _cast(delta, io_dtype), _cast(z, io_dtype), dirs,
                      io_dtype, bc_dtype)


def config_inputs(cfg_index: int, k: int = 0, a_init: str = "s4d") -> ScanInputs:
    """Inputs of config ``cfg_index`` drawn with seed ``1000*cfg_index + k``; A by
    the workloads' recipe (S4D-real) unless ``a_init="random"``."""
    c = CONFIGS[cfg_index]
    return make_inputs(c.batch, c.dim, c.len, dstate=c.dstate, bidir=c.bidir, io_dtype=c.io_dtype,
                       bc_dtype=c.bc_dtype, seed=config_seed(cfg_index, k), dt_range=c.dt_range, a_init=a_init)


def f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact float64 copy of a CPU tensor (bf16 and f32 widen exactly)."""
    if t is None:
        return None
    return np.ascontiguousarray(t.detach().to("cpu", torch.float64).numpy())


def as_f64_dict(x: ScanInputs) -> Dict[str, object]:
    """Float64 numpy views of every input, for the oracle."""
    return {
        "u": f64(x.u), "delta": f64(x.delta), "z": f64(x.z),
        "dirs": [dict(delta_bias=f64(p.delta_bias), A=f64(p.A), B=f64(p.B), C=f64(p.C), D=f64(p.D))
                 for p in x.dirs],
    }
