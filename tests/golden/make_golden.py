"""Writes trimul_n4_c6.json: a tiny regression fixture for the oracle.

The pages print no worked example for the triangle multiplicative update, so
this fixture is not a pin against the pages: its expected values come from the
oracle's scalar-loop spelling (oracle.bruteforce) only, on inputs drawn here
with numpy.  It guards the vectorised oracle against drift.  Run from the repo
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import bruteforce  # noqa: E402


def main():
    r = np.random.default_rng(2024)
    n, c_z, c = 4, 6, 4
    w = {
        "w_a_proj": r.standard_normal((c, c_z)) * 0.4, "w_a_gate": r.standard_normal((c, c_z)) * 0.4,
        "w_b_proj": r.standard_normal((c, c_z)) * 0.4, "w_b_gate": r.standard_normal((c, c_z)) * 0.4,
        "w_out_gate": r.standard_normal((c_z, c_z)) * 0.4, "w_out_proj": r.standard_normal((c_z, c)) * 0.5,
        "ln_in_w": 1 + 0.1 * r.standard_normal(c_z), "ln_in_b": 0.1 * r.standard_normal(c_z),
        "ln_out_w": 1 + 0.1 * r.standard_normal(c), "ln_out_b": 0.1 * r.standard_normal(c),
    }
    z = r.standard_normal((n, n, c_z))
    m = (r.random((n, n)) < 0.75).astype(int)
    g = {"about": __doc__.strip().splitlines()[0], "n": n, "c_z": c_z, "c": c,
         "weights": {k: v.tolist() for k, v in w.items()}, "z": z.tolist(), "mask": m.tolist()}
    for d in ("outgoing", "incoming"):
        g["out_" + d] = bruteforce.trimul_loops(z.tolist(), m.tolist(), w, d)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "trimul_n4_c6.json")
    with open(path, "w") as f:
        json.dump(g, f, indent=0)


if __name__ == "__main__":
    main()
