"""The fp64 oracle against stored 60-digit values (tests/golden/mp_tiny.json,
written by tests/golden/make_golden.py from the oracle package's mpmath
evaluation of the materialised form; see that file's "source" field)."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mp_tiny.json")


def test_oracle_matches_golden_mp_values(oracle_lib):
    doc = json.load(open(GOLDEN))
    x = doc["inputs"]
    u, z, delta = (np.array(x[k]) for k in ("u", "z", "delta"))
    f, r = [{k: np.array(v) for k, v in p.items()} for p in x["dirs"]]
    f["delta"] = r["delta"] = delta
    exp = {k: np.array([[[float(s) for s in row] for row in plane] for plane in v])
           for k, v in doc["expected"].items()}
    fwd = oracle_lib.sscan_fwd(u, delta, f["A"], f["B"], f["C"], f["D"], z, f["delta_bias"])
    rev = oracle_lib.sscan_fwd(u, delta, r["A"], r["B"], r["C"], r["D"], z, r["delta_bias"], reverse=True)
    bid = oracle_lib.sscan_bidir(u, z, f, r)
    for got, key in ((fwd, "fwd"), (rev, "rev"), (bid, "bidir")):
        ref = exp[key]
        np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15 * np.abs(ref).max())
