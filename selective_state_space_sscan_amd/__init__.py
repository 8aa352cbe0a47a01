"""MI355X (gfx950) selective scan (Mamba S6): C-ABI library + thin Python binding.

``fwd`` / ``bidir`` call ``libsscan.so`` (``selective_scan`` /
``selective_scan_bidir``: the same with gradients through the backward entry points) (build it with
``python -m selective_state_space_sscan_amd.build``); ``inputs`` draws the seeded
synthetic workloads.
"""
from .sscan import (SSCAN_BF16, SSCAN_F32, SScanError, bidir, fwd, load_library, run_inputs,  # noqa: F401
                    selective_scan, selective_scan_bidir, strerror, workspace_bytes)

__all__ = ["fwd", "bidir", "run_inputs", "workspace_bytes", "load_library", "strerror", "SScanError",
           "SSCAN_F32", "SSCAN_BF16", "selective_scan", "selective_scan_bidir"]
