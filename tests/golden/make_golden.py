"""Writes the stored expected values of ``mp_tiny.json``.

Calls only the oracle package (its mpmath evaluation of the materialised form,
Hand-written simplified Mamba2 page, section 3.1) on inputs from the shared seeded
generator, so no expected value comes from the GPU path.  Run from the repository
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import brute  # noqa: E402
from selective_state_space_sscan_amd.inputs import as_f64_dict, make_inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mp_tiny.json")


def main():
    x = as_f64_dict(make_inputs(1, 2, 6, dstate=4, bidir=True, seed=7, a_init="s4d"))
    f, r = [dict(p, delta=x["delta"]) for p in x["dirs"]]
    cases = {}
    for name, dirs, rev in (("fwd", [f], False), ("rev", [r], True), ("bidir", [f, r], False)):
        y = brute.brute_mp(x["u"], x["z"], dirs, reverse_single=rev, dps=60)
        cases[name] = [[[repr(float(v)) for v in row] for row in plane] for plane in y]
    tolist = lambda a: np.asarray(a).tolist()
    doc = {
        "what": "gated selective-scan outputs of a tiny case, 60-digit mpmath evaluation of the "
                "materialised (dual) form, rounded to float64",
        "source": "Hand-written simplified Mamba2 page sections 2.2, 3.1, 4.4; Reproducing Vision Mamba "
                  "page section 3.2 (bidirectional sum before the gate)",
        "generator": "selective_state_space_sscan_amd.inputs.make_inputs(1, 2, 6, dstate=4, bidir=True, seed=7, a_init='s4d')",
        "softplus": True,
        "inputs": {"u": tolist(x["u"]), "delta": tolist(x["delta"]), "z": tolist(x["z"]),
                   "dirs": [{k: tolist(v) for k, v in p.items()} for p in x["dirs"]]},
        "expected": cases,
    }
    with open(OUT, "w") as fh:
        json.dump(doc, fh, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
