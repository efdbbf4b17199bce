"""The allocation kernel's search, modelled on the CPU and held against the oracle.

`allocate_kernel` does not run the greedy step by step: it finds the B-th item
of the greedy's order (gain desc, channel asc, plane asc) with two short
bitwise searches, first the item's level (the double exponent of w_c 4^(-t),
halved), then, among the channels with an item at that level, the r largest
fraction-and-channel keys.  This file restates those two searches in numpy,
exactly as the kernel orders its comparisons, and checks the depths they give
against ``oracle.fathom_oracle.waterfill_depths`` (the greedy written out) on
random importances with zeros, exact ties, subnormal products and every kind
of budget.  It pins the search's design; the GPU parity tests pin the kernel.
"""

import numpy as np
import pytest

from oracle.fathom_oracle import waterfill_depths


def level_fraction_depths(w32: np.ndarray, budget: int) -> np.ndarray:
    d = w32.size
    x = (w32.astype(np.float64).view(np.uint64) >> np.uint64(29)).astype(np.int64)
    pos = w32 > 0
    lvl = np.where(pos, x >> 24, 0)
    key = ((x & 0xFFFFFF) << 8) | (255 - np.arange(d))
    nz = 4 * int(pos.sum())
    if budget == 0:
        return np.zeros(d, np.int64)
    if budget > nz:
        # nonzero channels read everything; zero channels fill in channel order
        rest = budget - nz
        zero = ~pos
        rank = np.cumsum(zero) - zero
        fill = np.minimum(rest - np.minimum(rest, 4 * rank), 4)
        return np.where(pos, 4, np.where(zero, fill, 0))

    def items_from(m):   # items of level >= m
        return int(np.clip(lvl - m + 1, 0, 4).sum())

    m = 0
    for bit in range(9, -1, -1):
        if items_from(m | (1 << bit)) >= budget:
            m |= 1 << bit
    r = budget - items_from(m + 1)
    cand = pos & (lvl - m >= 0) & (lvl - m <= 3)
    T = 0
    for bit in range(31, -1, -1):
        if int((cand & (key >= (T | (1 << bit)))).sum()) >= r:
            T |= 1 << bit
    chosen = cand & (key >= T)
    return np.where(pos, np.clip(lvl - m, 0, 4) + chosen, 0)


def importances(rng, d, kind):
    q = rng.standard_normal(d).astype(np.float32)
    s2 = np.exp(rng.standard_normal(d)).astype(np.float32)
    if kind == "zeros":
        q[rng.random(d) < 0.3] = 0
    elif kind == "ties":
        q = np.where(rng.random(d) < 0.5, np.float32(0.5), np.float32(-0.5)).astype(np.float32)
        s2[:] = 1
    elif kind == "tiny":
        q = (rng.standard_normal(d) * 1e-20).astype(np.float32)   # q^2 subnormal or zero
    elif kind == "prefix":
        q[:] = 0
        q[: rng.integers(0, d + 1)] = 1.0
    # the kernel's importance: two fp32 products, never fused
    return ((q * q).astype(np.float32) * s2).astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "zeros", "ties", "tiny", "prefix"])
def test_level_fraction_search_equals_the_greedy(kind):
    rng = np.random.default_rng([7, len(kind)])
    for _ in range(80):
        d = int(rng.choice([4, 5, 64, 100, 128, 256]))
        w = importances(rng, d, kind)
        for budget in (0, 1, int(rng.integers(0, 4 * d + 1)), 4 * d - 1, 4 * d):
            budget = max(0, budget)
            assert np.array_equal(level_fraction_depths(w, budget),
                                  waterfill_depths(w.astype(np.float64), budget)), (kind, d, budget)
