"""Pins of the oracle's reconstruction, scores and top-k selection.

Fathom digest (Method, key modules 4-5 and Output): a rule on the read prefix
rebuilds each channel's value, the scan scores every key and outputs the top-k
indices per query.  Review "Strengths" (paper Sec 3.3): every extra bit cuts
the channel's error by 4x.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import fathom_oracle as O
from tests.exact import fr


def case(seed, n=1500, d=32, g=4):
    rng = np.random.default_rng(seed)
    sigma = np.exp(rng.standard_normal(d)).astype(np.float32)
    k = rng.standard_normal((n, d)).astype(np.float32) * sigma
    q = rng.standard_normal((g, d)).astype(np.float32)
    return k, q, (sigma * sigma).astype(np.float32)


def test_full_budget_scores_equal_dequant_matmul():
    """B = 4d reads every plane: scores are q . dequant(K) with dequant = (kappa - 7.5) Delta."""
    k, q, s2 = case(1)
    delta, kappa, _ = O.pack_head(k)
    n, d = k.shape
    blk = np.arange(n) // 128
    deq = (kappa.astype(np.float64) - 7.5) * delta[:, blk].T.astype(np.float64)
    for h in range(q.shape[0]):
        t = O.waterfill_depths(O.importance(q[h], s2), 4 * d)
        assert np.all(t == 4)
        s, a = O.scores(q[h], kappa, delta, t)
        ref = deq @ q[h].astype(np.float64)
        assert np.allclose(s, ref, rtol=0, atol=1e-12 * np.max(a))
        assert np.allclose(a, np.abs(deq) @ np.abs(q[h].astype(np.float64)), rtol=1e-13)


def test_scores_exact_against_fractions():
    """fp64 scores agree with exact rational sums to ~1e-15 of sum |q k_hat|."""
    k, q, s2 = case(2, n=300, d=12)
    delta, kappa, _ = O.pack_head(k)
    t = O.waterfill_depths(O.importance(q[0], s2), 20)
    s, a = O.scores(q[0], kappa, delta, t)
    for j in range(0, 300, 7):
        tot = Fraction(0)
        for c in range(12):
            tc = int(t[c])
            if tc == 0:
                continue
            dl = fr(delta[c, j // 128])
            step = dl * 2 ** (4 - tc)
            kh = step * ((int(kappa[j, c]) >> (4 - tc)) - Fraction(2 ** (tc - 1)) + Fraction(1, 2))
            tot += fr(q[0, c]) * kh
        assert abs(fr(s[j]) - tot) <= Fraction(1, 10 ** 14) * fr(a[j]) + Fraction(1, 10 ** 300)


@pytest.mark.parametrize("budget", [0, 10, 46, 64, 92, 128])
def test_error_bound_per_bit(budget):
    """|s(t) - s(4)| <= sum_c |q_c| Delta_c (2^(4-t_c) - 1) / 2: the t-bit cell
    midpoint is within half the coarse cell minus half the fine cell of the
    4-bit midpoint."""
    k, q, s2 = case(3)
    delta, kappa, _ = O.pack_head(k)
    n, d = k.shape
    blk = np.arange(n) // 128
    full = np.full(d, 4)
    for h in range(q.shape[0]):
        t = O.waterfill_depths(O.importance(q[h], s2), budget)
        s, _ = O.scores(q[h], kappa, delta, t)
        s4, _ = O.scores(q[h], kappa, delta, full)
        bound = (np.abs(q[h].astype(np.float64))[None, :] * delta[:, blk].T.astype(np.float64)
                 * (2.0 ** (4 - t) - 1) / 2).sum(axis=1)
        assert np.all(np.abs(s - s4) <= bound * (1 + 1e-12) + 1e-300)


def test_four_x_per_bit_mse():
    """Midpoint reconstruction of a t-bit prefix has mean squared error
    (2^(4-t) Delta)^2 / 12 for keys uniform over the code range: each extra
    plane divides the error by 4."""
    delta = np.float16(0.5)
    m = 1 << 14
    x = ((np.arange(m) + 0.5) / m * 16 - 8).astype(np.float64) * float(delta)   # uniform grid
    xk = x.astype(np.float32)
    kappa = np.clip(np.floor(x / float(delta)) + 8, 0, 15).astype(np.uint8)
    mse = []
    for t in range(0, 5):
        kh = O.reconstruct(kappa, t, np.full(m, delta))
        mse.append(np.mean((kh - xk.astype(np.float64)) ** 2))
    for t in range(0, 5):
        assert math.isclose(mse[t], (2.0 ** (4 - t) * float(delta)) ** 2 / 12, rel_tol=1e-6)
    for t in range(4):
        assert math.isclose(mse[t] / mse[t + 1], 4.0, rel_tol=1e-6)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(30):
        n = int(rng.integers(1, 200))
        s = rng.integers(-5, 6, n).astype(np.float64)
        if trial % 4 == 0:
            s[rng.integers(0, n, 3)] = -0.0
        for k in sorted({0, 1, n // 2, n}):
            want = sorted(sorted(range(n), key=lambda j: (-s[j], j))[:k])
            assert list(O.topk(s, k)) == want


def test_topk_signed_zero_ties_by_index():
    s = np.array([0.0, -0.0, 0.0, -1.0, -0.0])
    assert list(O.topk(s, 2)) == [0, 1]
    assert list(O.topk(s, 4)) == [0, 1, 2, 4]


def test_step_matches_pure_python_pipeline():
    """Whole step (quantise, allocate, score, select) at tiny size against a
    pure-Python, exact-rational re-derivation that shares nothing with the
    oracle but the definitions."""
    rng = np.random.default_rng(12)
    h_kv, g, n, d = 2, 2, 260, 6
    k = (rng.standard_normal((h_kv, n, d)) * 2).astype(np.float32)
    q = rng.standard_normal((h_kv * g, d)).astype(np.float32)
    s2 = np.exp(rng.standard_normal((h_kv, d))).astype(np.float32)
    budget, kk = 9, 7
    res = O.step(k, q, s2, budget, kk)
    from tests.exact import F16, F32, round_binary
    for kv in range(h_kv):
        nb = (n + 127) // 128
        dl = [[round_binary(max(abs(fr(k[kv, j, c])) for j in range(b * 128, min(n, b * 128 + 128))) / 8, *F16)
               for b in range(nb)] for c in range(d)]
        code = [[8 if dl[c][j // 128] == 0 else min(15, max(0, math.floor(fr(k[kv, j, c]) / dl[c][j // 128]) + 8))
                 for c in range(d)] for j in range(n)]
        for h in range(kv * g, kv * g + g):
            w = [round_binary(round_binary(fr(q[h, c]) ** 2, *F32) * fr(s2[kv, c]), *F32) for c in range(d)]
            t = [0] * d
            for _ in range(budget):
                best = None
                for c in range(d):
                    if t[c] < 4 and (best is None or w[c] / 4 ** t[c] > w[best] / 4 ** t[best]):
                        best = c
                t[best] += 1
            assert list(res["depth"][h]) == t
            sc = []
            for j in range(n):
                tot = Fraction(0)
                for c in range(d):
                    if t[c]:
                        step_ = dl[c][j // 128] * 2 ** (4 - t[c])
                        tot += fr(q[h, c]) * step_ * ((code[j][c] >> (4 - t[c])) - Fraction(2 ** (t[c] - 1)) + Fraction(1, 2))
                sc.append(tot)
            want = sorted(sorted(range(n), key=lambda j: (-sc[j], j))[:kk])
            assert list(res["idx"][h]) == want
        assert list(res["union"][kv]) == [max(res["depth"][h][c] for h in range(kv * g, kv * g + g)) for c in range(d)]


# ---- appending keys: sealed blocks plus an exact open tail ----

def test_tail_scores_are_exact_rational_sums():
    from fractions import Fraction
    rng = np.random.default_rng(31)
    q = (rng.standard_normal(16) * 3).astype(np.float32)
    tk = (rng.standard_normal((5, 16)) * np.exp(rng.standard_normal((5, 16)))).astype(np.float32)
    s, a = O.tail_scores(q, tk)
    for j in range(5):
        exact = sum(Fraction(float(q[c])) * Fraction(float(tk[j, c])) for c in range(16))
        asum = sum(abs(Fraction(float(q[c])) * Fraction(float(tk[j, c]))) for c in range(16))
        assert abs(Fraction(s[j]) - exact) <= asum * Fraction(1, 2 ** 48)
        assert abs(Fraction(a[j]) - asum) <= asum * Fraction(1, 2 ** 48)


def test_step_append_with_empty_tail_is_step():
    rng = np.random.default_rng(32)
    kk = rng.standard_normal((2, 384, 32)).astype(np.float32)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    s2 = np.exp(rng.standard_normal((2, 32))).astype(np.float32)
    a = O.step(kk, q, s2, 40, 50)
    b = O.step_append(kk, np.zeros((2, 0, 32), np.float32), q, s2, 40, 50)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["depth"], b["depth"])
    for h in range(4):
        assert np.array_equal(a["scores"][h], b["scores"][h])


def test_step_append_all_tail_is_exact_topk():
    rng = np.random.default_rng(33)
    tk = rng.standard_normal((1, 100, 16)).astype(np.float32)
    q = rng.standard_normal((2, 16)).astype(np.float32)
    r = O.step_append(np.zeros((1, 0, 16), np.float32), tk, q, np.ones((1, 16), np.float32), 20, 10)
    for h in range(2):
        s = [sum(float(q[h, c]) * float(tk[0, j, c]) for c in range(16)) for j in range(100)]
        want = sorted(sorted(range(100), key=lambda j: (-s[j], j))[:10])
        assert list(r["idx"][h]) == want


def test_step_append_tail_indices_follow_the_sealed_keys():
    rng = np.random.default_rng(34)
    kk = rng.standard_normal((1, 256, 8)).astype(np.float32) * np.float32(0.01)
    tk = np.full((1, 3, 8), 50.0, np.float32)           # tail keys dominate every score
    q = np.ones((1, 8), np.float32)
    r = O.step_append(kk, tk, q, np.ones((1, 8), np.float32), 32, 3)
    assert list(r["idx"][0]) == [256, 257, 258]
