"""Builds ``libsscan.so`` (C ABI + gfx950 kernels) in-tree with hipcc.

Run ``python -m selective_state_space_sscan_amd.build`` from the repository root
(or call ``build()``).  hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsscan.so")

SOURCES = ["sscan_kernels.hip", "sscan_short.hip", "sscan_bwd.hip", "sscan_conv_bwd.hip", "sscan_multi.hip", "sscan_noalloc.hip", "sscan_capi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


OBJ_DIR = os.path.join(ROOT, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 target feature and says so; harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def _deps(src: str) -> set:
    """``src`` and the local headers it includes (``#include "..."``), transitively."""
    import re

    seen, todo = set(), [src]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(f):
            continue
        seen.add(f)
        with open(f) as fh:
            for name in re.findall(r'^\s*#\s*include\s+"([^"]+)"', fh.read(), re.M):
                todo += [os.path.join(d, name) for d in (CSRC, INCLUDE)]
    return seen


def _stale(obj: str, src: str) -> bool:
    """True when ``obj`` is missing or older than its source or a header it includes."""
    if not os.path.exists(obj):
        return True
    return max(os.path.getmtime(d) for d in _deps(src)) > os.path.getmtime(obj)


def build(verbose: bool = False, force: bool = True) -> str:
    """Compile the sources (in parallel, into _build/) and link ``libsscan.so``
    next to this file; returns its path.  ``force=False`` recompiles only the
    objects older than their source or a header."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJ_DIR, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if not force and not _stale(obj, os.path.join(CSRC, src)):
            continue
        cmds.append([hipcc()] + compile_flags + ["-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, os.path.join(CSRC, src)])
    with ThreadPoolExecutor(max(1, min(len(cmds), os.cpu_count() or 1))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, force="--changed" not in sys.argv))
