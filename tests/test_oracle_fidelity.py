"""The fidelity report's harness: when k = n every mode keeps every key, so
recall is 1 and the attention error is exactly 0; metrics stay in range at a
small k; the floor row is the exact top-k."""

import numpy as np

from tests import fidelity_report as R


def test_every_mode_is_exact_when_k_equals_n():
    for label, bits, rec, err in R.measure(n=1024, kv_heads=1, k=1024):
        assert np.all(rec == 1.0), label
        assert np.all(err == 0.0), label


def test_metrics_in_range_at_small_k():
    res = R.measure(n=4096, kv_heads=1, k=64)
    assert res[0][0].startswith("exact") and np.all(res[0][2] == 1.0)
    assert len(res) == len(R.MODES) + 1
    for label, bits, rec, err in res:
        assert rec.shape == (4,) and err.shape == (4,)
        assert np.all((rec >= 0) & (rec <= 1)), label
        assert np.all(np.isfinite(err) & (err >= 0)), label
    # the 68- and 136-bit fixed modes read 17 and 34 channels of 4 planes
    assert [b for _, b, _, _ in res[1:]] == [46, 68, 92, 512, 92, 68, 136, 68, 136]
