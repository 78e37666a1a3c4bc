"""Distance measures used to compare results against the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/zero_oracle.py).

ulp distance: bit patterns are mapped to integers that are ordered like the
values they encode (non-negative floats keep their magnitude bits, negative
floats map to minus their magnitude bits, so +0 and -0 both map to 0), and the
distance is the absolute difference.  Two NaNs are at distance 0; a NaN and a
non-NaN are at distance INF_ULP.
"""
from __future__ import annotations

import numpy as np

INF_ULP = np.iinfo(np.int64).max


def _ordered(bits: np.ndarray, sign_bit: int, mag_mask: int) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & mag_mask
    return np.where(b & sign_bit, -mag, mag)


def _dist(a_bits, b_bits, a_nan, b_nan, sign_bit, mag_mask):
    d = np.abs(_ordered(a_bits, sign_bit, mag_mask) - _ordered(b_bits, sign_bit, mag_mask))
    d = np.where(a_nan & b_nan, 0, d)
    d = np.where(a_nan ^ b_nan, INF_ULP, d)
    return d


def ulp_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    assert a.shape == b.shape
    return _dist(a.view(np.uint32), b.view(np.uint32), np.isnan(a), np.isnan(b),
                 0x80000000, 0x7FFFFFFF)


def ulp_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a_bits).view(np.uint16)
    b = np.ascontiguousarray(b_bits).view(np.uint16)
    assert a.shape == b.shape
    a_nan = (a & 0x7FFF) > 0x7F80
    b_nan = (b & 0x7FFF) > 0x7F80
    return _dist(a, b, a_nan, b_nan, 0x8000, 0x7FFF)


def max_ulp_f32(a, b) -> int:
    return int(ulp_f32(a, b).max(initial=0))


def max_ulp_bf16(a, b) -> int:
    return int(ulp_bf16(a, b).max(initial=0))


def bits_equal_f32(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit-exact equality, except that any two NaNs compare equal."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    if a.shape != b.shape:
        return False
    same = a.view(np.uint32) == b.view(np.uint32)
    same |= np.isnan(a) & np.isnan(b)
    return bool(same.all())
