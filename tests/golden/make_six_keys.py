"""Writes six_keys.json: a six-key, two-channel worked example through the oracle.

The pages refer to a six-key worked example (review, "Strengths", paper App. A)
whose numbers are not in the text; this is our own example of the same size,
chosen so every value can be checked by hand (see six_keys.md).  Calls only
oracle/.  Run from the repository root:  python tests/golden/make_six_keys.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import fathom_oracle as O  # noqa: E402

K = np.array([[8.0, 0.25], [-4.0, -2.0], [2.0, 1.0], [-1.0, 1.5], [0.5, -0.75], [6.0, 0.0]], np.float32)
Q = np.array([1.0, 2.0], np.float32)
S2 = np.array([1.0, 1.0], np.float32)

delta, kappa, rec = O.pack_head(K)
out = {"keys": K.tolist(), "q": Q.tolist(), "sigma2": S2.tolist(),
       "delta": [float(x) for x in delta[:, 0]],
       "kappa": kappa.T.tolist(),
       "records_hex": [bytes(r).hex() for r in rec],
       "budgets": {}}
w = O.importance(Q, S2)
for b in range(0, 9):
    t = O.waterfill_depths(w, b)
    s, a = O.scores(Q, kappa, delta, t)
    out["budgets"][str(b)] = {"depth": [int(x) for x in t], "scores": [float(x) for x in s],
                              "sums": [float(x) for x in a], "top2": [int(x) for x in O.topk(s, 2)]}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "six_keys.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
print("wrote", path)
