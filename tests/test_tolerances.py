"""The attention acceptance bound itself (a test criterion, CPU only)."""

import numpy as np

from oracle import attention_oracle as A
from synthetic import to_bf16_bits
from tests.tolerances import attention_tolerance


def rows(rng, n, d):
    return to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))


def test_tolerance_is_positive_and_scales_with_the_values():
    rng = np.random.default_rng(7)
    kr, vr = rows(rng, 200, 64), rows(rng, 200, 64)
    q = rng.standard_normal(64).astype(np.float32)
    idx = np.arange(0, 200, 3)
    t1, l1 = attention_tolerance(q, kr, vr, idx, 0.125)
    vr2 = to_bf16_bits(A.bf16_to_f64(vr).astype(np.float32) * np.float32(4))
    t2, _ = attention_tolerance(q, kr, vr2, idx, 0.125)
    assert np.all(t1 > 0) and l1 > 0
    np.testing.assert_allclose(t2, 4 * t1, rtol=1e-12)
    assert np.all(t1 < 1e-3)


def test_default_bound_does_not_depend_on_a_kernel_structure():
    """The default chains are the list length and d + 2: looser than any
    shorter structural chain, and growing with the list, not with a split
    count."""
    rng = np.random.default_rng(8)
    kr, vr = rows(rng, 600, 128), rows(rng, 600, 128)
    q = rng.standard_normal(128).astype(np.float32)
    idx = np.arange(0, 600, 2)
    t_any, l_any = attention_tolerance(q, kr, vr, idx, 0.09)
    t_str, l_str = attention_tolerance(q, kr, vr, idx, 0.09, logit_chain=26, sum_chain=32)
    assert np.all(t_str < t_any) and l_str < l_any
    t_same, _ = attention_tolerance(q, kr, vr, idx, 0.09, logit_chain=130, sum_chain=idx.size)
    np.testing.assert_array_equal(t_same, t_any)


def test_empty_list_has_zero_tolerance():
    rng = np.random.default_rng(9)
    kr, vr = rows(rng, 10, 16), rows(rng, 10, 16)
    t, l = attention_tolerance(rng.standard_normal(16).astype(np.float32), kr, vr, np.array([-1, 10]), 0.5)
    assert np.all(t == 0) and l == 0.0
