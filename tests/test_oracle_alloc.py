"""Pins of the oracle's per-query read-depth allocation.

Sources: the Fathom arXiv abstract and the ai-feeds digest (Method, key module
2) describe the allocation as reverse water-filling of the per-key bit budget
over channel importance q_c^2 sigma_c^2; the evolve.pub review, "Strengths"
(paper Sec 3.3), gives the reason for the rule: one more plane divides a
channel's squared error by 4.  Objective: minimise sum_c w_c 4^(-t_c) subject
to sum_c t_c = B, t_c in {0..4}.
"""

import itertools
import zlib
from fractions import Fraction

import numpy as np
import pytest

from oracle import fathom_oracle as O
from tests.exact import F32, fr, round_binary


def objective(w, t) -> Fraction:
    return sum(fr(w[c]) * Fraction(1, 4 ** int(t[c])) for c in range(len(w)))


def random_weights(rng, d, kind):
    if kind == "lognormal":
        w = np.exp(rng.standard_normal(d) * 2).astype(np.float32)
    elif kind == "ties":
        w = rng.choice(np.array([0.0, 1.0, 4.0, 16.0, 0.25], np.float32), d)
    elif kind == "zeros":
        w = np.zeros(d, np.float32)
        w[rng.integers(0, d)] = np.float32(3.0)
    else:
        w = rng.integers(0, 5, d).astype(np.float32) * np.float32(0.5)
    return w.astype(np.float32)


def test_importance_rounding_exact():
    rng = np.random.default_rng(1)
    q = (rng.standard_normal(300) * np.exp(rng.standard_normal(300) * 3)).astype(np.float32)
    s2 = np.exp(rng.standard_normal(300) * 3).astype(np.float32)
    w = O.importance(q, s2)
    for c in range(300):
        qq = round_binary(fr(q[c]) * fr(q[c]), *F32)
        want = round_binary(qq * fr(s2[c]), *F32)
        assert fr(w[c]) == want


def test_importance_rejects_bad_inputs():
    with pytest.raises(ValueError):
        O.importance(np.array([np.nan], np.float32), np.ones(1, np.float32))
    with pytest.raises(ValueError):
        O.importance(np.ones(1, np.float32), np.array([-1.0], np.float32))
    with pytest.raises(ValueError):
        O.importance(np.array([1e30], np.float32), np.ones(1, np.float32))


@pytest.mark.parametrize("kind", ["lognormal", "ties", "zeros", "halves"])
def test_greedy_equals_brute_force_d4(kind):
    """Greedy reaches the exact minimum over all 5^4 depth vectors for every B <= 16,
    and equals the minimiser whenever it is unique."""
    rng = np.random.default_rng(zlib.crc32(kind.encode()))   # fixed per kind, not per process
    cands = list(itertools.product(range(5), repeat=4))
    for trial in range(40):
        w = random_weights(rng, 4, kind)
        for b in range(0, 17):
            t = O.waterfill_depths(w, b)
            assert int(t.sum()) == b and t.min() >= 0 and t.max() <= 4
            feas = [c for c in cands if sum(c) == b]
            vals = [objective(w, c) for c in feas]
            best = min(vals)
            assert objective(w, t) == best
            argmins = [c for c, v in zip(feas, vals) if v == best]
            if len(argmins) == 1:
                assert tuple(int(x) for x in t) == argmins[0]


def greedy_by_sorted_gains(w, b):
    """Independent formulation of the same rule: list every (channel, plane) gain
    w_c 4^-t, order by (gain desc, channel asc, plane asc), take the first B."""
    items = []
    for c in range(len(w)):
        for t in range(4):
            items.append((-(fr(w[c]) / 4 ** t), c, t))
    items.sort()
    depth = [0] * len(w)
    for _, c, _ in items[:b]:
        depth[c] += 1
    return depth


@pytest.mark.parametrize("kind", ["lognormal", "ties", "zeros", "halves"])
def test_greedy_tie_break_matches_sorted_gain_rule(kind):
    rng = np.random.default_rng(3 + len(kind))
    for trial in range(10):
        w = random_weights(rng, 24, kind)
        for b in (0, 1, 5, 17, 46, 95, 96):
            assert list(O.waterfill_depths(w, b)) == greedy_by_sorted_gains(w, b)


def test_sum_and_exchange_certificate_d128():
    """sum t = B, and no single-bit move improves: for c with t_c < 4 and c' with
    t_c' > 0, w_c 4^-t_c <= w_c' 4^-(t_c'-1), equality only when c' < c (the
    lower channel took the tied bit)."""
    rng = np.random.default_rng(9)
    for trial in range(6):
        q = rng.standard_normal(128).astype(np.float32)
        s2 = np.exp(rng.standard_normal(128)).astype(np.float32)
        if trial % 2:
            s2[rng.choice(128, 4, replace=False)] *= np.float32(100.0)
        w = O.importance(q, s2)
        for b in (0, 1, 46, 64, 68, 92, 136, 300, 511, 512):
            t = O.waterfill_depths(w, b)
            assert int(t.sum()) == b
            nxt = {c: fr(w[c]) / 4 ** int(t[c]) for c in range(128) if t[c] < 4}
            last = {c: fr(w[c]) / 4 ** (int(t[c]) - 1) for c in range(128) if t[c] > 0}
            for c, gn in nxt.items():
                for c2, gl in last.items():
                    if c2 == c:
                        continue
                    assert gn < gl or (gn == gl and c2 < c), (b, c, c2)


def test_monotone_in_budget():
    """The greedy is incremental: t(B+1) - t(B) is one unit vector."""
    rng = np.random.default_rng(21)
    w = O.importance(rng.standard_normal(128).astype(np.float32), np.exp(rng.standard_normal(128)).astype(np.float32))
    prev = O.waterfill_depths(w, 0)
    for b in range(1, 513):
        cur = O.waterfill_depths(w, b)
        diff = cur - prev
        assert diff.min() == 0 and diff.sum() == 1
        prev = cur


def test_water_level_closed_form():
    """Reverse water-filling picture: with distinct gains, channel c gets
    t_c = #{t in 0..3 : w_c 4^-t >= level}, where level is the B-th largest of all
    gains w_c 4^-t (the water level)."""
    rng = np.random.default_rng(31)
    w = np.exp(rng.standard_normal(128) * 2).astype(np.float32)
    gains = sorted((fr(w[c]) / 4 ** t for c in range(128) for t in range(4)), reverse=True)
    for b in (1, 20, 92, 200, 511):
        level = gains[b - 1]
        want = [sum(1 for t in range(4) if fr(w[c]) / 4 ** t >= level) for c in range(128)]
        assert list(O.waterfill_depths(w, b)) == want


def test_budget_extremes():
    w = np.arange(1, 9, dtype=np.float32)
    assert list(O.waterfill_depths(w, 0)) == [0] * 8
    assert list(O.waterfill_depths(w, 32)) == [4] * 8
    # all-zero importance: every gain ties at 0 -> lowest channels fill first
    assert list(O.waterfill_depths(np.zeros(4, np.float32), 6)) == [4, 2, 0, 0]
    with pytest.raises(ValueError):
        O.waterfill_depths(w, 33)


def test_topq_matches_selection_loop():
    rng = np.random.default_rng(4)
    for trial in range(20):
        q = rng.standard_normal(128).astype(np.float32)
        if trial % 3 == 0:
            q[rng.choice(128, 20)] = np.float32(0.5)     # ties in |q|
            q[rng.choice(128, 10)] = np.float32(-0.5)
        for m in (0, 1, 17, 34, 128):
            chosen, left = [], list(range(128))
            for _ in range(m):
                best = left[0]
                for c in left:
                    if abs(fr(q[c])) > abs(fr(q[best])):
                        best = c
                chosen.append(best)
                left.remove(best)
            want = [4 if c in chosen else 0 for c in range(128)]
            assert list(O.topq_depths(q, m)) == want


def test_union_contains_every_prefix():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    s2 = np.exp(rng.standard_normal(128)).astype(np.float32)
    dep = np.stack([O.waterfill_depths(O.importance(q[h], s2), 92) for h in range(4)])
    u = O.union_depths(dep)
    assert np.all(u >= dep) and np.all((u[None] == dep).any(axis=0))


# ---- group-shared allocation (one depth vector per KV head) ----

def test_group_importance_of_one_head_is_importance():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 128)).astype(np.float32)
    s2 = np.exp(rng.standard_normal(128)).astype(np.float32)
    assert np.array_equal(O.group_importance(q, s2), O.importance(q[0], s2))


def test_group_importance_is_sequential_fp32_sum():
    rng = np.random.default_rng(22)
    qs = (rng.standard_normal((4, 64)) * np.exp(rng.standard_normal((4, 64)) * 2)).astype(np.float32)
    s2 = np.exp(rng.standard_normal(64) * 2).astype(np.float32)
    got = O.group_importance(qs, s2)
    for c in range(64):
        acc = Fraction(0)
        for h in range(4):
            w = round_binary(round_binary(fr(qs[h, c]) * fr(qs[h, c]), *F32) * fr(s2[c]), *F32)
            acc = round_binary(acc + w, *F32)
        assert fr(got[c]) == acc


def test_group_allocation_minimises_the_summed_objective_d4():
    """With weights whose fp32 sums are exact (small dyadic values), the shared
    depth vector minimises sum_h sum_c w_hc 4^-t_c over all 5^4 vectors."""
    rng = np.random.default_rng(23)
    cands = list(itertools.product(range(5), repeat=4))
    for trial in range(30):
        qs = rng.integers(-3, 4, (4, 4)).astype(np.float32) * np.float32(0.5)
        s2 = rng.choice(np.array([0.25, 1.0, 2.0, 4.0], np.float32), 4)
        wh = [O.importance(qs[h], s2) for h in range(4)]
        wg = O.group_importance(qs, s2)
        for b in range(0, 17):
            t = O.waterfill_depths(wg, b)
            assert int(t.sum()) == b

            def obj(c):
                return sum(objective(wh[h], c) for h in range(4))
            feas = [c for c in cands if sum(c) == b]
            vals = [obj(c) for c in feas]
            assert obj(t) == min(vals)


def test_static_matches_selection_loop():
    rng = np.random.default_rng(41)
    for trial in range(20):
        s2 = np.exp(rng.standard_normal(128)).astype(np.float32)
        if trial % 3 == 0:
            s2[rng.choice(128, 20)] = np.float32(2.0)      # ties
            s2[rng.choice(128, 10)] = np.float32(0.0)      # zero variance
        if trial % 3 == 1:
            s2[rng.choice(128, 12)] = np.float32(-0.0)     # -0 ranks as 0 (lowest channel first)
            s2[rng.choice(128, 6)] = np.float32(0.0)
        for m in (0, 1, 17, 34, 128):
            chosen, left = [], list(range(128))
            for _ in range(m):
                best = left[0]
                for c in left:
                    if fr(s2[c]) > fr(s2[best]):
                        best = c
                chosen.append(best)
                left.remove(best)
            want = [4 if c in chosen else 0 for c in range(128)]
            assert list(O.static_depths(s2, m)) == want
