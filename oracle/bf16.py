"""bfloat16 helpers: raw bits <-> float64, and direct float64 -> bf16 rounding.

bfloat16 = 1 sign, 8 exponent (bias 127), 7 mantissa bits; the top half of an
IEEE binary32. Rounding to bf16 here is done once, directly from float64
(round to nearest, ties to even; overflow to infinity), so there is no double
rounding through float32.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np


def to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float32 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def to_f64(bits) -> np.ndarray:
    return to_f32(bits).astype(np.float64)


def round_from_f64(values) -> np.ndarray:
    """float64 -> bf16 bits (uint16), round to nearest even, single rounding."""
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, a)
    _, k = np.frexp(a)
    floor_log2 = k.astype(np.int64) - 1
    # 8 significant bits in the normal range; fixed spacing 2^-133 below 2^-126.
    step_exp = np.maximum(floor_log2, -126) - 7
    n = np.rint(np.ldexp(a, -step_exp))
    y = np.ldexp(n, step_exp)
    overflow = y >= 2.0 ** 128
    y32 = np.where(overflow, 0.0, y).astype(np.float32)  # exact: y is a bf16 value
    bits = (y32.view(np.uint32) >> 16).astype(np.uint32)
    bits = np.where(overflow, 0x7F80, bits)
    bits = np.where(nan, 0x7FC0, bits)
    bits = bits | (neg.astype(np.uint32) << 15)
    return bits.astype(np.uint16)


def ulp(bits) -> np.ndarray:
    """Spacing of bf16 values at each (finite) bf16 value, as float64."""
    v = np.abs(to_f64(bits))
    _, k = np.frexp(v)
    floor_log2 = np.where(v > 0, k.astype(np.int64) - 1, -126)
    return np.ldexp(1.0, np.maximum(floor_log2, -126) - 7)
