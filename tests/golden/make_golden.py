"""Writes tests/golden/gdn2_tiny.json: a tiny fixed example evaluated by the fp64 oracle.

The pages print no worked numeric example of the recurrence (burn-gdn2 0.1.5 docs page,
section "Architecture", gives only the equation), so this fixture is not a value from the
pages: it freezes the oracle's own fp64 output on hand-picked inputs (d_k=3, d_v=2, four
tokens, negative-eigenvalue erase gate, nonzero S0) so that any later change to the
oracle's arithmetic shows up as a failing test. Only ``oracle`` is called.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

INPUTS = {
    "q": [[0.6, 0.0, 0.8], [0.0, 1.0, 0.0], [0.48, 0.6, 0.64], [-0.8, 0.6, 0.0]],
    "k": [[1.0, 0.0, 0.0], [0.6, 0.8, 0.0], [0.0, 0.6, -0.8], [0.36, 0.48, 0.8]],
    "v": [[1.0, -2.0], [0.5, 0.25], [-1.5, 3.0], [2.0, 0.0]],
    "w": [[0.5, 0.75], [1.0, 0.25], [0.125, 0.5], [0.875, 0.625]],
    "log_alpha": [[-0.5, -0.25, -1.0], [-0.125, -2.0, -0.75], [-0.0625, -0.5, -1.5],
                  [-1.25, -0.375, -0.25]],
    "b": [[1.5, 0.25, 1.0], [0.5, 1.75, 0.125], [1.0, 1.0, 1.9], [0.05, 0.6, 1.2]],
    "S0": [[0.1, -0.2], [0.3, 0.05], [-0.4, 0.2]],
}


def main():
    x = {n: np.array(v, dtype=np.float64) for n, v in INPUTS.items()}
    o, ST = oracle.recurrent(x["q"][:, None], x["k"][:, None], x["v"][:, None],
                             x["log_alpha"][:, None], x["b"][:, None], x["w"][:, None],
                             S0=x["S0"][None, None])
    out = {"source": "fp64 oracle (oracle.recurrent) on the inputs below; regression fixture",
           "inputs": INPUTS, "o": o[:, 0].tolist(), "S_T": ST[0, 0].tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gdn2_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
