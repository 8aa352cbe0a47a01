"""HBM traffic of the scan kernels from rocprofv3 counter collections.

``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report, per dispatch, the
KiB the L2 read from / wrote to memory.  Both are scaled by what the same counter
reads for a plain streaming kernel of known traffic (bench.py --copy-calibration
negates 512 MiB: 512 MiB read, 512 MiB written): the factor is known bytes /
counted bytes.  The summary is keyed by the
SHA-256 of the kernel sources, so a summary taken before the kernels changed is
recognisably stale.

  python -m selective_state_space_sscan_amd.profiling FETCH_DIR WRITE_DIR OUT.json

FETCH_DIR / WRITE_DIR are the rocprofv3 output directories (containing
*counter_collection.csv) of ``bench.py --copy-calibration`` runs.

VALU issue of the same kernels, from one ``rocprofv3 --pmc VALUBusy SQ_WAVES
SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32`` run of bench.py (MeanOccupancyPerCU may be
added to the same pass):

  python -m selective_state_space_sscan_amd.profiling valu SQ_DIR OUT.json

gives per kernel the VALUBusy percentage, the VALU instructions per wave (and the
share of transcendentals), the waves per launch and, when counted, the mean number
of resident waves per compute unit, keyed by the same source hash.
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
COPY_BYTES = 512 << 20
COPY_KERNEL = "neg_kernel"  # the calibration kernel (torch.neg), unique in the run
KERNELS = {"stage_bc_kernel": "stage_bc", "scan_aggregate_kernel": "aggregate", "scan_carry_kernel": "carry",
           "scan_output_dir_kernel": "output", "scan_output_bidir_kernel": "output",
           "scan_short_quad_kernel": "output"}


# the files that define the forward scan's kernels (staging, aggregate, carry, output)
FORWARD_SOURCES = ("sscan_device.h", "sscan_internal.h", "sscan_kernels.hip", "sscan_short.hip")


def kernel_source_hash() -> str:
    """SHA-256 over the forward kernels' source files (name and contents)."""
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _rows(directory: str):
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    for f in files:
        for r in csv.DictReader(open(f)):
            yield f, r


def _per_dispatch(directory: str, counter: str):
    """{step name or 'copy': mean counter value (KiB) per dispatch}."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    total = collections.defaultdict(float)
    dispatches = collections.defaultdict(set)
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = "copy" if COPY_KERNEL in name else next((v for k, v in KERNELS.items() if k in name), None)
            if key is None:
                continue
            total[key] += float(r["Counter_Value"])
            dispatches[key].add((f, r["Dispatch_Id"]))
    return {k: total[k] / len(dispatches[k]) for k in total}


def summarize(fetch_dir: str, write_dir: str) -> dict:
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / (fetch["copy"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy"] * 1024.0)
    steps = {}
    for k in fetch:
        if k == "copy":
            continue
        rd = fetch[k] * 1024.0 * f_scale
        wr = write.get(k, 0.0) * 1024.0 * w_scale
        steps[k] = {"read_bytes": rd, "write_bytes": wr, "bytes": rd + wr}
    return {"kernel_source_sha256": kernel_source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
            "copy_bytes": COPY_BYTES, "per_launch": steps}


VALU_COUNTERS = ("VALUBusy", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "MeanOccupancyPerCU")


def summarize_valu(sq_dir: str) -> dict:
    """Per scan kernel: mean VALUBusy (%), waves per launch, VALU and
    transcendental instructions per wave, over the launches of one counter run."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    seen = collections.defaultdict(set)  # counters present per kernel
    for f, r in _rows(sq_dir):
        key = next((v for k, v in KERNELS.items() if k in r["Kernel_Name"]), None)
        if key is None or r["Counter_Name"] not in VALU_COUNTERS:
            continue
        vals[key][r["Counter_Name"]] += float(r["Counter_Value"])
        seen[key].add(r["Counter_Name"])
        disp[key].add((f, r["Dispatch_Id"]))
    out = {}
    for k, v in vals.items():
        n = len(disp[k])
        waves = v["SQ_WAVES"] / n
        out[k] = {"valu_busy_pct": v["VALUBusy"] / n, "waves_per_launch": waves,
                  "valu_insts_per_wave": v["SQ_INSTS_VALU"] / v["SQ_WAVES"] if v["SQ_WAVES"] else None,
                  "trans_share": v["SQ_INSTS_VALU_TRANS_F32"] / v["SQ_INSTS_VALU"] if v["SQ_INSTS_VALU"] else None,
                  "launches": n}
        if "MeanOccupancyPerCU" in seen[k]:
            out[k]["mean_occupancy_per_cu"] = v["MeanOccupancyPerCU"] / n
    return {"kernel_source_sha256": kernel_source_hash(), "per_launch": out}


def load_traffic(path: str):
    """The per-launch traffic summary if it matches the current kernel source, else None."""
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    if doc.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return doc


load_valu = load_traffic  # the same staleness rule (kernel source hash)


if __name__ == "__main__":
    if len(sys.argv) == 4 and sys.argv[1] == "valu":
        doc = summarize_valu(sys.argv[2])
    elif len(sys.argv) == 4:
        doc = summarize(sys.argv[1], sys.argv[2])
    else:
        sys.exit(__doc__)
    with open(sys.argv[3], "w") as fh:
        json.dump(doc, fh, indent=1)
    print(json.dumps(doc, indent=1))
