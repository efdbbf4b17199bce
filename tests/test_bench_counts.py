"""The figures bench.py divides by time to place the scan on its roofline: the
algorithmic bytes of a step (the union prefix runs) against the oracle's record
layout, and the operation count against a hand count on small depth tables."""

import importlib.util
import os

import numpy as np
import pytest

from oracle import fathom_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("n", [128, 1000, 1024, 4096, 131072, 1 << 20, 3 * 1024 + 300])
def test_algorithmic_bytes_are_the_prefix_runs(bench, n):
    rng = np.random.default_rng(n)
    union = rng.integers(0, 5, size=(3, 17)).astype(np.uint8)
    want = sum(O.prefix_bytes(n, int(t)) for t in union.ravel())
    assert bench.algorithmic_bytes(union, n) == want


def test_algorithmic_ops_hand_count(bench):
    # one KV head, two query heads, four channels
    depth = np.array([[0, 1, 2, 4],
                      [0, 3, 2, 1]], np.uint8)
    union = depth.max(axis=0)[None]                  # [0, 3, 2, 4]
    n = 256                                          # two 128-key blocks
    # per 4 keys: 2 ops per union plane: 2 * (0 + 3 + 2 + 4) = 18
    # 5 per distinct depth in use per channel: 5 * (0 + 2 + 1 + 2) = 25
    # 4 fmas per reading head: 4 * (0 + 2 + 2 + 2) = 24
    assert bench.algorithmic_ops(depth, union, n) == (18 + 25 + 24) * (n // 4)


def test_algorithmic_ops_of_an_empty_budget(bench):
    depth = np.zeros((4, 8), np.uint8)
    assert bench.algorithmic_ops(depth, depth.max(axis=0)[None], 1024) == 0
    assert bench.algorithmic_bytes(depth.max(axis=0)[None], 1024) == 0
