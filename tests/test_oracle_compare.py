"""Pins for the distance measures every parity test goes through
(oracle/compare.py): ulp distance on binary32 and bfloat16 bit patterns and
bit-exact equality.

The sharded owners must end a step holding one and the same model (slide
"分担数据，与分担保存责任，是两个动作", note 原 N48: the owners' updated slices
together form the same new version), and the GPU-against-oracle checks of that
claim are only as strong as these measures.  Every value below is fixed by
hand from the IEEE 754 encodings (binary32: 1 sign, 8 exponent, 23 fraction
bits; bfloat16: the upper 16 bits of a binary32), not by re-running the
measures' own formula:

* adjacent representable values are 1 apart, on both sides of zero;
* +0 and -0 are the same value, at distance 0;
* the two smallest subnormals of opposite sign are 2 apart (-d, then 0, then +d);
* the largest finite value and infinity are adjacent;
* within one binade of binary32 there are 2^23 values, so [1, 2) spans 2^23;
* any two NaNs are at distance 0, a NaN and a non-NaN at INF_ULP;
* bfloat16 0x7F80 is +infinity and 0x7F81..0x7FFF are NaNs.

A stepping pin counts the representable values between two floats with
numpy's nextafter, one at a time, which shares nothing with the bit mapping.
"""
import numpy as np
import pytest

from oracle.compare import (INF_ULP, bits_equal_f32, max_ulp_bf16, max_ulp_f32, ulp_bf16,
                            ulp_f32)

F32 = np.float32


def f32_bits(u):
    return np.array([u], dtype=np.uint32).view(np.float32)


def d32(a, b):
    return int(ulp_f32(np.asarray([a], F32), np.asarray([b], F32))[0])


def d32b(ua, ub):
    """Distance between two binary32 values given as bit patterns."""
    return int(ulp_f32(f32_bits(ua), f32_bits(ub))[0])


def d16(ua, ub):
    return int(ulp_bf16(np.array([ua], np.uint16), np.array([ub], np.uint16))[0])


MIN_SUB = 0x00000001       # smallest positive subnormal
MIN_NORMAL = 0x00800000
MAX_FINITE = 0x7F7FFFFF
INF = 0x7F800000
QNAN = 0x7FC00000
ONE = 0x3F800000


# ---------------------------------------------------------------- binary32, hand-fixed values
@pytest.mark.parametrize("ua, ub, want", [
    (ONE, ONE + 1, 1),                        # 1 and the next float up
    (ONE, ONE - 1, 1),                        # 1 and the next float down (previous binade)
    (0x00000000, 0x80000000, 0),              # +0, -0
    (MIN_SUB, 0x80000000 | MIN_SUB, 2),       # +d, -d: -d, -0 = +0, +d
    (0x00000000, MIN_SUB, 1),
    (0x80000000, MIN_SUB, 1),                 # -0 and +d
    (0x80000000 | MIN_SUB, 2 * MIN_SUB, 3),   # -d and +2d
    (MIN_NORMAL - 1, MIN_NORMAL, 1),          # largest subnormal, smallest normal
    (MAX_FINITE, INF, 1),                     # largest finite and +inf
    (0x80000000 | MAX_FINITE, 0x80000000 | INF, 1),
    (INF, 0x80000000 | INF, 2 * INF),         # +inf and -inf: every finite value lies between
    (ONE, 0x40000000, 1 << 23),               # 1.0 and 2.0: one binade
    (0x80000000 | ONE, ONE, 2 * ONE),         # -1 and +1
    (0x40400000, 0x40400000, 0),              # 3.0 and itself
])
def test_ulp_f32_hand_fixed(ua, ub, want):
    assert d32b(ua, ub) == want
    assert d32b(ub, ua) == want


@pytest.mark.parametrize("nan_a, nan_b", [(QNAN, QNAN), (QNAN, 0x7F800001), (0xFFC00000, 0x7FFFFFFF),
                                          (0x7FA00000, 0xFF800001)])
def test_ulp_f32_two_nans_are_equal(nan_a, nan_b):
    assert d32b(nan_a, nan_b) == 0


@pytest.mark.parametrize("nan", [QNAN, 0x7F800001, 0xFFFFFFFF])
@pytest.mark.parametrize("other", [0x00000000, 0x80000000, ONE, INF, 0x80000000 | INF, MAX_FINITE, MIN_SUB])
def test_ulp_f32_nan_against_a_number_is_infinite(nan, other):
    assert d32b(nan, other) == INF_ULP
    assert d32b(other, nan) == INF_ULP


def test_ulp_f32_elementwise_and_max():
    a = np.array([1.0, 0.0, np.nan, 2.0], F32)
    b = np.array([np.nextafter(F32(1), F32(2)), -0.0, np.nan, 2.0], F32)
    assert ulp_f32(a, b).tolist() == [1, 0, 0, 0]
    assert max_ulp_f32(a, b) == 1
    assert max_ulp_f32(np.zeros(0, F32), np.zeros(0, F32)) == 0
    b[3] = np.nan
    assert max_ulp_f32(a, b) == INF_ULP


def test_ulp_f32_counts_floats_by_stepping():
    # between x and y (x < y) the distance is the number of nextafter steps
    # from x to y (stepping up from -d gives -0, then +d: zero is one value)
    rng = np.random.default_rng(7)
    starts = [F32(1.0), F32(-1.0), F32(3.0e-38), F32(-1e-44), F32(0.0), F32(-0.0),
              F32(-1.4e-45), np.nextafter(F32(np.inf), F32(0))]
    starts += [F32(x) for x in rng.normal(0, 1e3, 6)]
    for x in starts:
        y, steps = x, 0
        for _ in range(300):
            with np.errstate(over="ignore"):
                y = np.nextafter(y, F32(np.inf))
            steps += 1
            if not np.isfinite(y):
                break
            if steps in (1, 2, 17, 128, 299):
                assert d32(x, y) == steps, (x, y, steps)
        assert d32(x, y) == steps


def test_ulp_f32_is_additive_along_sorted_values():
    # the ordered map is monotone: for a <= b <= c, d(a, c) = d(a, b) + d(b, c)
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0xFFFFFFFF, size=3000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = np.sort(x[np.isfinite(x)])
    a, b, c = x[:-2], x[1:-1], x[2:]
    assert np.array_equal(ulp_f32(a, c), ulp_f32(a, b) + ulp_f32(b, c))


# ---------------------------------------------------------------- bfloat16, hand-fixed values
@pytest.mark.parametrize("ua, ub, want", [
    (0x3F80, 0x3F81, 1),            # 1.0 and the next bf16 up
    (0x3F80, 0x3F7F, 1),
    (0x0000, 0x8000, 0),            # +0, -0
    (0x0001, 0x8001, 2),            # smallest subnormals of opposite sign
    (0x7F7F, 0x7F80, 1),            # largest finite and +inf: 0x7F80 is not a NaN
    (0xFF7F, 0xFF80, 1),
    (0x3F80, 0x4000, 128),          # 1.0 and 2.0: 2^7 values per binade
    (0xBF80, 0x3F80, 2 * 0x3F80),
    (0x7F80, 0xFF80, 2 * 0x7F80),
])
def test_ulp_bf16_hand_fixed(ua, ub, want):
    assert d16(ua, ub) == want
    assert d16(ub, ua) == want


@pytest.mark.parametrize("nan", [0x7F81, 0x7FC0, 0x7FFF, 0xFF81, 0xFFC0])
def test_ulp_bf16_nans(nan):
    assert d16(nan, 0x7FC0) == 0
    assert d16(nan, 0xFFFF) == 0
    for other in (0x7F80, 0xFF80, 0x0000, 0x3F80, 0x7F7F):
        assert d16(nan, other) == INF_ULP
        assert d16(other, nan) == INF_ULP


def test_ulp_bf16_agrees_with_binary32_on_the_upper_half():
    # a bf16 pattern is the upper half of a binary32 whose lower half is zero;
    # binary32 distances between such values are 2^16 times the bf16 distance
    rng = np.random.default_rng(11)
    a = rng.integers(0, 1 << 16, 5000).astype(np.uint16)
    b = rng.integers(0, 1 << 16, 5000).astype(np.uint16)
    fa = (a.astype(np.uint32) << 16).view(np.float32)
    fb = (b.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(fa) | np.isnan(fb)
    d_bf = ulp_bf16(a, b)
    d_32 = ulp_f32(fa, fb)
    assert np.array_equal(d_bf[~nan] << 16, d_32[~nan])
    assert np.array_equal(d_bf[nan], d_32[nan])
    assert max_ulp_bf16(a[:0], b[:0]) == 0


# ---------------------------------------------------------------- bit-exact equality
def test_bits_equal_f32():
    a = np.array([1.0, -2.5, 0.0, np.inf], F32)
    assert bits_equal_f32(a, a.copy())
    assert not bits_equal_f32(np.array([0.0], F32), np.array([-0.0], F32))
    assert not bits_equal_f32(np.array([1.0], F32), np.array([np.nextafter(F32(1), F32(2))], F32))
    assert bits_equal_f32(f32_bits(QNAN), f32_bits(0xFFC00001))      # any two NaNs
    assert not bits_equal_f32(f32_bits(QNAN), f32_bits(INF))
    assert not bits_equal_f32(np.zeros(3, F32), np.zeros(4, F32))
    assert bits_equal_f32(np.zeros(0, F32), np.zeros(0, F32))
