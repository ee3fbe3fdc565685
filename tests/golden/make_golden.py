"""Write the frozen fp32 Lloyd-Max table fixture from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
The table is the fp32 rounding of the double-precision Lloyd-Max fixed point
for N(0, 1) (PolyKV explainer, section 2.B: precomputed Lloyd-Max centroids
for N(0, 1)); thresholds are midpoints computed in double before rounding.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import lloyd_max  # noqa: E402


def hex32(a):
    return [format(int(x), "08x") for x in np.asarray(a, dtype=np.float32).view(np.uint32)]


def main():
    out = {"source": "oracle.lloyd_max.table_f32 (written by tests/golden/make_golden.py)", "tables": {}}
    for b in (2, 3, 4):
        c, t = lloyd_max.table_f32(b)
        out["tables"][str(b)] = {
            "centroids_hex": hex32(c),
            "thresholds_hex": hex32(t),
            "centroids": [float(x) for x in c],
            "thresholds": [float(x) for x in t],
        }
    with open(os.path.join(HERE, "lloyd_max_fp32.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
