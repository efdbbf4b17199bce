"""Pins of the oracle's quantiser and record packer against exact arithmetic.

Source: the evolve.pub review, "Strengths" (paper Sec 3.2) and FAQ.  Keys are
quantised to 4-bit uniform codes with one scale per block and kept per channel
as bit planes; reading the top t planes of a code yields the t-bit mid-rise
quantiser of the same value, which these pins check.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import fathom_oracle as O
from tests.exact import F16, fr, round_binary


def exact_scale(values) -> Fraction:
    m = max(abs(fr(v)) for v in values)
    return round_binary(m / 8, *F16)


def exact_code(x, delta: Fraction) -> int:
    if delta == 0:
        return 8
    return min(15, max(0, math.floor(fr(x) / delta) + 8))


def crafted_keys():
    """Keys with exact threshold hits, clamping, zero, tiny and subnormal-scale blocks."""
    n, d = 5 * 128 + 37, 6          # ragged: 5 full blocks + a 37-key tail
    rng = np.random.default_rng(7)
    k = rng.standard_normal((n, d)).astype(np.float32)
    k *= np.float32(3.0)
    # channel 0, block 0: max |k| = 8 -> Delta = 1; threshold hits and neighbours
    blk = np.zeros(128, np.float32)
    vals = [8.0, -8.0, 3.0, -3.0, 0.0, -0.0, 0.5, -0.5, 7.0, -7.0, 6.999999523, -6.999999523,
            1.0, np.nextafter(np.float32(1.0), np.float32(0)), np.nextafter(np.float32(-1.0), np.float32(0))]
    blk[: len(vals)] = np.array(vals, np.float32)
    k[:128, 0] = blk
    # channel 1, block 1: max/8 = 1 + 2^-11 -> ties to even -> Delta = 1, and 8(1+2^-11) clamps to 15
    k[128:256, 1] = np.linspace(-4, 4, 128).astype(np.float32)
    k[130, 1] = np.float32(8.0 * (1 + 2.0 ** -11))
    # channel 2, block 2: all zeros -> Delta = 0 -> code 8
    k[256:384, 2] = 0.0
    # channel 3, block 3: tiny -> Delta underflows to 0 in fp16 -> code 8 although keys are nonzero
    k[384:512, 3] = rng.standard_normal(128).astype(np.float32) * np.float32(1e-9)
    # channel 4, block 4: scale is an fp16 subnormal
    k[512:640, 4] = rng.standard_normal(128).astype(np.float32) * np.float32(1e-6)
    # channel 5: large values (scale near the top of fp16)
    k[:, 5] *= np.float32(1.0e4)
    return k


def test_scales_and_codes_match_exact_floor():
    k = crafted_keys()
    n, d = k.shape
    delta = O.block_scales(k)
    kappa = O.quantize_codes(k, delta)
    assert delta.shape == (d, O.n_blocks(n)) and kappa.shape == (n, d)
    for c in range(d):
        for b in range(O.n_blocks(n)):
            lo, hi = b * 128, min(n, (b + 1) * 128)
            ds = exact_scale(k[lo:hi, c])
            assert fr(delta[c, b]) == ds, (c, b)
            for j in range(lo, hi):
                assert kappa[j, c] == exact_code(k[j, c], ds), (j, c)


def test_hand_worked_block():
    # channel 0, block 0 of crafted_keys: Delta = 1 exactly
    k = crafted_keys()
    delta = O.block_scales(k)
    kappa = O.quantize_codes(k, delta)
    assert float(delta[0, 0]) == 1.0
    # 8 -> floor 8 + 8 = 16 -> clamp 15; -8 -> 0; 3 -> 11; -3 -> 5; 0 and -0 -> 8;
    # 0.5 -> 8; -0.5 -> 7; 7 -> 15; -7 -> 1; 6.9999995 -> 14; -6.9999995 -> 1;
    # 1 -> 9; just below 1 -> 8; just above -1 -> 7
    expect = [15, 0, 11, 5, 8, 8, 8, 7, 15, 1, 14, 1, 9, 8, 7]
    assert list(kappa[: len(expect), 0]) == expect
    # max/8 = 1 + 2^-11 is halfway between fp16 1 and 1 + 2^-10: ties to even -> 1
    assert float(delta[1, 1]) == 1.0 and kappa[130, 1] == 15
    assert float(delta[2, 2]) == 0.0 and np.all(kappa[256:384, 2] == 8)
    assert float(delta[3, 3]) == 0.0 and np.all(kappa[384:512, 3] == 8)
    assert 0 < float(delta[4, 4]) < 2.0 ** -14          # subnormal fp16 scale


@pytest.mark.parametrize("t", [1, 2, 3, 4])
def test_prefix_is_t_bit_midrise_quantizer(t):
    """kappa >> (4-t) equals the t-bit mid-rise quantizer with step 2^(4-t) Delta,
    and the oracle's reconstruction is the midpoint of that quantizer's cell."""
    rng = np.random.default_rng(11 + t)
    n = 2048
    k = (rng.standard_normal((n, 1)) * 2.5).astype(np.float32)
    k[::97] = np.float32(0.0)
    delta = O.block_scales(k)
    kappa = O.quantize_codes(k, delta)
    for j in range(n):
        dl = fr(delta[0, j // 128])
        step = dl * 2 ** (4 - t)
        code_t = min(2 ** t - 1, max(0, math.floor(fr(k[j, 0]) / step) + 2 ** (t - 1)))
        assert (int(kappa[j, 0]) >> (4 - t)) == code_t
        lo_edge = (code_t - 2 ** (t - 1)) * step
        hi_edge = lo_edge + step
        mid = (lo_edge + hi_edge) / 2
        kh = O.reconstruct(kappa[j:j + 1, 0], t, delta[0, j // 128:j // 128 + 1])[0]
        assert fr(kh) == mid


def test_nesting_exhaustive_codes():
    """For every 4-bit code and depth t, the t-bit prefix cell contains the 4-bit cell."""
    delta = np.array([np.float16(0.375)])
    for code in range(16):
        fine_lo = (code - 8) * Fraction(3, 8)
        fine_hi = fine_lo + Fraction(3, 8)
        for t in range(1, 5):
            step = Fraction(3, 8) * 2 ** (4 - t)
            pref = code >> (4 - t)
            lo = (pref - 2 ** (t - 1)) * step
            assert lo <= fine_lo and fine_hi <= lo + step
            kh = O.reconstruct(np.array([code], np.uint8), t, delta)[0]
            assert fr(kh) == lo + step / 2


def test_four_plane_prefix_is_full_dequant():
    """Reading all 4 planes reconstructs (kappa - 7.5) * Delta (full 4-bit dequantisation)."""
    rng = np.random.default_rng(3)
    k = (rng.standard_normal((1024, 8)) * np.exp(rng.standard_normal(8))).astype(np.float32)
    delta = O.block_scales(k)
    kappa = O.quantize_codes(k, delta)
    blk = np.arange(1024) // 128
    for c in range(8):
        full = (kappa[:, c].astype(np.float64) - 7.5) * delta[c, blk].astype(np.float64)
        assert np.array_equal(O.reconstruct(kappa[:, c], 4, delta[c, blk]), full)
        assert np.array_equal(O.reconstruct(kappa[:, c], 0, delta[c, blk]), np.zeros(1024))


def test_record_layout_bit_by_bit():
    """Decode records byte by byte from the layout definition (no numpy bit helpers):
    unit u of the head holds the fp16 scales of blocks 8u..8u+7 then the plane-0
    bits of keys 1024u..1024u+1023; planes 1-3 follow, one bit per key."""
    k = crafted_keys()
    n, d = k.shape
    delta, kappa, rec = O.pack_head(k)
    u, h, p, r = O.record_layout(n)
    nb = O.n_blocks(n)
    assert rec.shape == (d, r) and h == 144 * u and p == 128 * u and r == h + 3 * p
    for c in range(d):
        raw = bytes(rec[c])
        for b in range(8 * u):
            (v,) = struct.unpack_from("<e", raw, 144 * (b // 8) + 2 * (b % 8))
            if b < nb:
                assert v == float(delta[c, b]) or (v == 0 and float(delta[c, b]) == 0)
            else:
                assert raw[144 * (b // 8) + 2 * (b % 8)] == 0 and raw[144 * (b // 8) + 2 * (b % 8) + 1] == 0
        for plane in range(4):
            for j in range(u * 1024):
                if plane == 0:
                    off = 144 * (j // 1024) + 16 + (j % 1024) // 8
                else:
                    off = h + (plane - 1) * p + j // 8
                bit = (raw[off] >> (j % 8)) & 1
                want = ((int(kappa[j, c]) >> (3 - plane)) & 1) if j < n else 0
                assert bit == want, (c, plane, j)


def test_record_sizes_and_prefix_runs():
    # n a multiple of 1024: R = n/64 + n/2 (scales, then four n/8-byte planes)
    for n in (4096, 131072, 262144, 1 << 20):
        u, h, p, r = O.record_layout(n)
        assert r == n // 64 + n // 2 and h == n // 64 + n // 8 and p == n // 8
        for t in range(5):
            assert O.prefix_bytes(n, t) == (0 if t == 0 else n // 64 + t * n // 8)
    assert O.record_layout(1) == (1, 144, 128, 528)
    assert O.record_layout(0) == (0, 0, 0, 0)


def test_unpack_roundtrip_and_prefix_read():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((777, 5)).astype(np.float32)
    delta, kappa, rec = O.pack_head(k)
    for t in range(0, 5):
        # only the prefix run is needed: clobber everything after it
        cut = rec.copy()
        cut[:, O.prefix_bytes(777, t):] = 0xA5
        d2, code = O.unpack_codes(cut, 777, t)
        if t:
            assert np.array_equal(d2.view(np.uint16), delta.view(np.uint16))
        assert np.array_equal(code, kappa >> (4 - t))


def test_invalid_keys_raise():
    k = np.zeros((128, 2), np.float32)
    k[3, 1] = np.nan
    with pytest.raises(ValueError):
        O.block_scales(k)
    k[3, 1] = np.float32(1e6)      # 1e6 / 8 = 125000 > fp16 max
    with pytest.raises(ValueError):
        O.block_scales(k)


# ---- the token-major 4-bit copy (the free path) ----

def test_nibbles_hand_example():
    kappa = np.array([[0, 15, 8, 3, 9], [1, 2, 14, 7, 12]])
    delta = np.array([[0.5], [1.0], [2.0], [0.25], [4.0]], np.float16)   # [d, n_blocks], as block_scales
    codes, scales = O.pack_nibbles(kappa, delta)
    # channel 0 low nibble, channel 1 high nibble of byte 0; the fifth channel
    # alone in byte 2 (high nibble 0)
    assert codes.tolist() == [[0xF0, 0x38, 0x09], [0x21, 0x7E, 0x0C]]
    assert codes.shape == (2, 3) and scales.shape == (1, 10)
    assert scales[0, :2].tolist() == [0x00, 0x38]        # fp16 0.5 = 0x3800, little-endian
    assert scales[0, 8:10].tolist() == [0x00, 0x44]      # fp16 4.0 = 0x4400


def test_nibbles_scales_follow_block_scales():
    rng = np.random.default_rng(52)
    k = (rng.standard_normal((300, 6)) * [1, 2, 4, 8, 16, 32]).astype(np.float32)
    delta = O.block_scales(k)                                     # [d, n_blocks] = [6, 3]
    _, scales = O.pack_nibbles(O.quantize_codes(k, delta), delta)
    got = scales.view("<f2").reshape(3, 6)                        # [n_blocks, d]
    assert np.array_equal(got.T.astype(np.float32), delta.astype(np.float32))


def test_nibbles_round_trip():
    rng = np.random.default_rng(51)
    for d in (1, 7, 64, 128):
        kappa = rng.integers(0, 16, (300, d))
        codes, _ = O.pack_nibbles(kappa, np.ones((d, 3), np.float16))
        assert codes.shape == (300, (d + 1) // 2)
        assert np.array_equal(O.unpack_nibbles(codes, d), kappa)
