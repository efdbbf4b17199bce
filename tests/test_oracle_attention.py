"""Pins of the sparse-attention oracle against facts that do not come from it:
hand-decoded bf16 patterns, dense softmax attention from scipy, exact rational
closed forms and invariances."""

from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import attention_oracle as A
from synthetic import to_bf16_bits

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rows(rng, n, d, scale=1.0):
    return to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32) * np.float32(scale))


def test_bf16_decode_hand_patterns():
    pats = np.array([0x3F80, 0xC000, 0x7F7F, 0x0001, 0x8000, 0x0000, 0x4049, 0x3E80], np.uint16)
    want = [1.0, -2.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, -0.0, 0.0,
            # 0x4049: sign 0, exponent 0x80 -> 2^1, mantissa 0x49 = 73 -> (1 + 73/128) * 2
            (1 + 73 / 128) * 2.0,
            # 0x3E80: exponent 0x7D -> 2^-2, mantissa 0
            0.25]
    got = A.bf16_to_f64(pats)
    assert list(got) == want
    assert np.signbit(got[4]) and not np.signbit(got[5])


def test_full_index_set_is_dense_softmax_attention():
    rng = np.random.default_rng(1)
    n, d = 300, 64
    kr, vr = rows(rng, n, d), rows(rng, n, d)
    q = rng.standard_normal(d).astype(np.float32)
    scale = 1 / np.sqrt(d)
    idx = np.arange(n)
    o, lse, p, valid = A.sparse_attention(q, kr, vr, idx, scale)
    kk, vv = A.bf16_to_f64(kr), A.bf16_to_f64(vr)
    s = np.float64(np.float32(scale)) * (kk @ q.astype(np.float64))
    ref_p = scipy.special.softmax(s)
    np.testing.assert_allclose(p, ref_p, rtol=1e-12, atol=0)
    np.testing.assert_allclose(o, ref_p @ vv, rtol=1e-11, atol=1e-13)
    assert abs(lse - scipy.special.logsumexp(s)) < 1e-12 * max(1.0, abs(lse))
    assert list(valid) == list(idx)


def test_single_key_gives_its_value_row():
    rng = np.random.default_rng(2)
    kr, vr = rows(rng, 50, 32), rows(rng, 50, 32)
    q = rng.standard_normal(32).astype(np.float32)
    o, lse, p, _ = A.sparse_attention(q, kr, vr, np.array([17]), 0.125)
    assert np.array_equal(o, A.bf16_to_f64(vr[17]))
    exact = Fraction(float(np.float32(0.125))) * sum(
        Fraction(float(qc)) * Fraction(float(kc)) for qc, kc in zip(q, A.bf16_to_f64(kr[17])))
    assert lse == float(exact) or abs(Fraction(lse) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
    assert list(p) == [1.0]


def test_zero_query_gives_the_mean_row_exactly():
    rng = np.random.default_rng(3)
    n, d = 40, 16
    kr, vr = rows(rng, n, d), rows(rng, n, d)
    idx = np.array([3, 9, 27, 31, 0])
    o, lse, p, _ = A.sparse_attention(np.zeros(d, np.float32), kr, vr, idx, 0.25)
    vals = A.bf16_to_f64(vr)
    for c in range(d):
        mean = sum(Fraction(float(vals[j, c])) for j in idx) / len(idx)
        assert abs(Fraction(o[c]) - mean) <= abs(mean) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)
    assert abs(lse - np.log(len(idx))) < 1e-15
    assert np.allclose(p, 1 / len(idx), rtol=1e-15)


def test_two_keys_follow_the_logistic_closed_form():
    d = 4
    one, two, half = 0x3F80, 0x4000, 0x3F00            # 1.0, 2.0, 0.5
    kr = np.array([[one, 0, 0, 0], [two, 0, 0, 0]], np.uint16)
    vr = np.array([[one, 0, two, 0], [0, one, 0, half]], np.uint16)
    q = np.array([1.5, 7.0, -3.0, 0.25], np.float32)
    o, lse, p, _ = A.sparse_attention(q, kr, vr, np.array([0, 1]), 1.0)
    a, b = 1.5, 3.0                                     # logits q . K_0, q . K_1
    w0 = 1 / (1 + np.exp(b - a))
    w1 = 1 / (1 + np.exp(a - b))
    np.testing.assert_allclose(p, [w0, w1], rtol=1e-15)
    np.testing.assert_allclose(o, [w0, w1, 2 * w0, 0.5 * w1], rtol=1e-15)
    np.testing.assert_allclose(lse, np.log(np.exp(a) + np.exp(b)), rtol=1e-15)


def test_order_of_the_index_set_does_not_matter():
    rng = np.random.default_rng(4)
    kr, vr = rows(rng, 500, 128, 3.0), rows(rng, 500, 128)
    q = rng.standard_normal(128).astype(np.float32)
    idx = rng.choice(500, 64, replace=False)
    o1, l1, _, _ = A.sparse_attention(q, kr, vr, idx, 0.0883883)
    o2, l2, _, _ = A.sparse_attention(q, kr, vr, idx[::-1].copy(), 0.0883883)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    assert abs(l1 - l2) < 1e-12


def test_huge_common_logit_does_not_overflow():
    # every row is a large common part plus a small distinct part; the result
    # must equal attention over the small parts (the common logit cancels)
    rng = np.random.default_rng(5)
    d = 8
    big = np.full((6, d), 0x4700, np.uint16)           # 32768.0 in every entry
    small = rows(rng, 6, d)
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    kr = big.copy()
    kr[:, 1:] = small[:, 1:]                            # channel 0 carries 32768 for all rows
    kr[:, 0] = 0x4700
    vr = rows(rng, 6, d)
    q2 = q.copy()
    q2[1] = 0.5
    o, lse, _, _ = A.sparse_attention(q2, kr, vr, np.arange(6), 1.0)
    kr_small = kr.copy()
    kr_small[:, 0] = 0
    o_ref, lse_ref, _, _ = A.sparse_attention(q2, kr_small, vr, np.arange(6), 1.0)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse - 32768.0, lse_ref, rtol=0, atol=1e-9)


def test_out_of_range_entries_are_skipped():
    rng = np.random.default_rng(6)
    n = 100
    kr, vr = rows(rng, n, 32), rows(rng, n, 32)
    q = rng.standard_normal(32).astype(np.float32)
    o1, l1, _, v1 = A.sparse_attention(q, kr, vr, np.array([5, -1, 40, n, 99, 1 << 40]), 0.2)
    o2, l2, _, v2 = A.sparse_attention(q, kr, vr, np.array([5, 40, 99]), 0.2)
    assert list(v1) == [5, 40, 99]
    assert np.array_equal(o1, o2) and l1 == l2
    o3, l3, p3, v3 = A.sparse_attention(q, kr, vr, np.array([-3, n]), 0.2)
    assert np.array_equal(o3, np.zeros(32)) and l3 == -np.inf and v3.size == 0


# ---- fidelity metrics --------------------------------------------------------

def test_recall_exact_fractions():
    exact = np.array([3, 10, 11, 40])
    assert A.topk_recall(exact, exact) == 1.0
    assert A.topk_recall(np.array([0, 1, 2, 5]), exact) == 0.0
    assert A.topk_recall(np.array([40, 0, 3, 7]), exact) == 0.5
    assert A.topk_recall(np.array([7, 3, 0, 40]), exact) == 0.5          # order does not matter
    assert A.topk_recall(np.array([11]), exact) == 0.25
    assert A.topk_recall(np.array([], dtype=np.int64), np.array([], dtype=np.int64)) == 1.0


def test_attention_error_is_zero_for_the_full_set_and_for_constant_values():
    rng = np.random.default_rng(8)
    n, d = 257, 32
    kr, vr = rows(rng, n, d), rows(rng, n, d)
    q = rng.standard_normal(d).astype(np.float32)
    assert A.attention_error(q, kr, vr, np.arange(n), 0.3) == 0.0
    const = np.tile(to_bf16_bits(rng.standard_normal(d).astype(np.float32)), (n, 1))
    for idx in (np.array([0]), np.arange(0, n, 7), np.array([n - 1, 5])):
        assert A.attention_error(q, kr, const, idx, 0.3) < 1e-15


def test_attention_error_two_keys_closed_form():
    rng = np.random.default_rng(9)
    d = 16
    kr, vr = rows(rng, 2, d), rows(rng, 2, d)
    q = rng.standard_normal(d).astype(np.float32)
    scale = 0.25
    kk, vv = A.bf16_to_f64(kr), A.bf16_to_f64(vr)
    p = scipy.special.softmax(scale * (kk @ q.astype(np.float64)))
    o = p[0] * vv[0] + p[1] * vv[1]
    want = p[1] * np.linalg.norm(vv[1] - vv[0]) / np.linalg.norm(o)
    got = A.attention_error(q, kr, vr, np.array([0]), scale)
    assert got == pytest.approx(want, rel=1e-12)


def test_attention_error_one_hot_values_at_zero_query():
    n, d = 96, 4
    kr = rows(np.random.default_rng(10), n, d)
    q = np.zeros(d, np.float32)                       # uniform weights 1/n
    for kept in ([0], [5, 17, 80], list(range(0, 96, 2)), list(range(95))):
        e0 = np.array([1, 0, 0, 0], np.float32)
        e1 = np.array([0, 1, 0, 0], np.float32)
        v = np.tile(e1, (n, 1))
        v[kept] = e0
        m = Fraction(len(kept), n)
        want = np.sqrt(2.0) * float(1 - m) / np.sqrt(float(m * m + (1 - m) * (1 - m)))
        got = A.attention_error(q, kr, to_bf16_bits(v), np.array(kept), 1.0)
        assert got == pytest.approx(want, rel=1e-13)
