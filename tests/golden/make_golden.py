"""Write tests/golden/oracle_small.json: a regression fixture for the fp64 oracle.

The pages ("Optimizing on-device inference for Apple Silicon") print no numeric example of
the recurrence, so no fixture here comes from them. This script calls only the oracle; the
values it stores are pinned by the closed forms and invariants in tests/oracle_pins.py
(run before regenerating), and the fixture guards the oracle against later regressions.
Inputs are small, hand-picked dyadic numbers so the case can be re-derived by hand.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402


def case():
    # n=1, t=3, h_qk=1, h_v=2, d_k=4, d_v=3
    q = np.array([[1, 0, 1, 0], [0.5, -1, 0, 2], [0, 0, -1, 1]], float).reshape(1, 3, 1, 4)
    k = np.array([[1, 1, 0, 0], [0, 1, -1, 0], [2, 0, 0, 1]], float).reshape(1, 3, 1, 4)
    v = np.array([[[1, -2, 0.5], [0, 1, 1]], [[0.25, 0, -1], [2, -1, 0]],
                  [[-1, 1, 1], [0.5, 0.5, -0.5]]], float).reshape(1, 3, 2, 3)
    g = np.array([[-0.5, -0.125], [0.0, -1.0], [-0.25, -0.0625]], float).reshape(1, 3, 2)
    beta = np.array([[0.5, 1.0], [0.75, 0.25], [1.0, 0.5]], float).reshape(1, 3, 2)
    s0 = (np.arange(2 * 4 * 3, dtype=float).reshape(1, 2, 4, 3) - 11.5) / 16.0
    return dict(q=q, k=k, v=v, g=g, beta=beta, state_in=s0, l2_eps=1e-6)


def main():
    c = case()
    out, st = oracle.run(c["q"], c["k"], c["v"], c["g"], c["beta"], c["state_in"],
                         l2_eps=c["l2_eps"], threads=1)
    doc = {"source": "tests/golden/make_golden.py (calls only oracle.run)",
           "inputs": {key: (val.tolist() if hasattr(val, "tolist") else val)
                      for key, val in c.items()},
           "out": out.tolist(), "state_out": st.tolist()}
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
