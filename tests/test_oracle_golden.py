"""The six-key worked example (tests/golden/six_keys.*) against the oracle and hand values."""

import json
import os

import numpy as np

from oracle import fathom_oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load():
    with open(os.path.join(HERE, "six_keys.json")) as f:
        return json.load(f)


def test_six_keys_fixture_reproduced():
    g = load()
    k = np.array(g["keys"], np.float32)
    q = np.array(g["q"], np.float32)
    s2 = np.array(g["sigma2"], np.float32)
    delta, kappa, rec = O.pack_head(k)
    assert [float(x) for x in delta[:, 0]] == g["delta"]
    assert kappa.T.tolist() == g["kappa"]
    assert [bytes(r).hex() for r in rec] == g["records_hex"]
    w = O.importance(q, s2)
    for b, v in g["budgets"].items():
        t = O.waterfill_depths(w, int(b))
        s, a = O.scores(q, kappa, delta, t)
        assert [int(x) for x in t] == v["depth"]
        assert [float(x) for x in s] == v["scores"]
        assert [int(x) for x in O.topk(s, 2)] == v["top2"]


def test_six_keys_hand_values():
    """Values derived by hand in six_keys.md."""
    g = load()
    assert g["delta"] == [1.0, 0.25]
    assert g["kappa"] == [[15, 4, 10, 7, 8, 14], [9, 0, 12, 14, 5, 8]]
    r0 = bytes.fromhex(g["records_hex"][0])
    assert r0[0:2] == b"\x00\x3c" and r0[16] == 0x35 and r0[144] == 0x2B
    depths = [g["budgets"][str(b)]["depth"] for b in range(1, 9)]
    assert depths == [[0, 1], [1, 1], [1, 2], [2, 2], [2, 3], [3, 3], [3, 4], [4, 4]]
    assert g["budgets"]["2"]["scores"] == [6.0, -6.0, 6.0, -2.0, 2.0, 6.0]
    assert g["budgets"]["2"]["top2"] == [0, 2]
    assert g["budgets"]["8"]["scores"][0] == 8.25
