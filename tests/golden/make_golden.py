"""Writes tests/golden/p3_formula_case.json from the fp64 oracle only.

Inputs: the deterministic demo inputs of page "flash-attention-v2-sram-tiling"
(aiqz.cc), section Python 演示: n=8, d=4, Q[i][t] = 0.5(i+1) + t,
K[i][t] = 0.3(i+1) - t, V[i][t] = 0.2(i+1) + 0.1t, scale 1/sqrt(d).  The page
prints no output values for this case, so the file is a regression lock on
the oracle, not a pin.
Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import ref  # noqa: E402


def main():
    n, d = 8, 4
    i = np.arange(n)[:, None] + 1.0
    t = np.arange(d)[None, :]
    q, k, v = i * 0.5 + t, i * 0.3 - t, i * 0.2 + 0.1 * t
    out = {"source": "page flash-attention-v2-sram-tiling (aiqz.cc), section Python 演示; values from oracle/ref.py",
           "scale": 0.5}
    for key, causal in (("full", False), ("causal", True)):
        o, lse, _, _ = ref.head_forward(q, k, v, 0.5, causal)
        out[key] = {"O": o.tolist(), "LSE": lse.tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "p3_formula_case.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
