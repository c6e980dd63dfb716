"""Writes tests/golden/oracle_tiny_f32.json from the fp64 oracle only.

The Ling & Ring 2.6 Technical Report pages print no values for the operator,
so this fixture is not a pin of the oracle; it freezes the oracle's output on
the tiny fp32 workload (B=1, H=2, N=256, d=64, seed 0) so that an accidental
change of the oracle or of the input recipe shows up as a diff.  The fixture
is regenerated only by running this script:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import la_inputs  # noqa: E402
import oracle  # noqa: E402

ROWS = [0, 1, 63, 64, 127, 200, 255]


def main():
    c = la_inputs.CONFIGS["tiny_f32"]
    q, k, v = la_inputs.qkv(c["seed"], c["B"], c["H"], c["N"], c["d"], dtype="f32")
    s = la_inputs.slopes(c["H"])
    o, S = oracle.fwd(q, k, v, s)
    out = {
        "workload": "tiny_f32 B=1 H=2 N=256 d=64 seed=0, q,k,v ~ N(0,1)/sqrt(d) fp32",
        "rows": ROWS,
        "o_rows": {str(h): o[0, h, ROWS].tolist() for h in range(c["H"])},
        "S_diag": {str(h): np.diag(S[0, h]).tolist() for h in range(c["H"])},
        "S_sum": [float(S[0, h].sum()) for h in range(c["H"])],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_f32.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
