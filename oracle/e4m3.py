"""OCP E4M3FN codec, written out from the format definition, in float64.

Format (the pages fix only "E4M3: 4-bit exponent and 3-bit mantissa" on all
tensors -- "Six Reasons Deepseek Ai Is A Waste Of Time", paragraph on the GEMM
operands; the Greek and Japanese codingmall.com pages, "unified E4M3 format").
The variant is OCP E4M3FN, the one gfx950's FP8 units use:

  code = s eeee mmm, exponent bias 7
  e == 0        : (-1)^s * (m / 8) * 2^-6          (subnormals, step 2^-9)
  1 <= e <= 15  : (-1)^s * (1 + m / 8) * 2^(e - 7)
  s 1111 111    : NaN (0x7F, 0xFF); there is no infinity; max finite 448 (0x7E)

Encoding rounds to nearest with ties to even at E4M3 precision, after clamping
the magnitude to 448 (saturation), and keeps the sign of zero.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6
SUBNORMAL_STEP_EXP = -9  # subnormal spacing 2^-9


def decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) as float64; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m, SUBNORMAL_STEP_EXP)
    mag = np.where(e == 0, subnormal, normal)
    out = sign * mag
    out = np.where((c & 0x7F) == 0x7F, np.nan, out)
    return out


def encode(values) -> np.ndarray:
    """E4M3 code of each float64 value: saturate to +-448, round to nearest even.

    The sign bit is the sign of the input, including for zero results. NaN
    inputs give the NaN code with the input's sign.
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, np.minimum(np.abs(v), MAX_FINITE))

    # Spacing of E4M3 values around a: 2^(floor(log2 a) - 3) in the normal
    # range, 2^-9 below 2^-6.
    _, k = np.frexp(a)  # a = f * 2^k with f in [0.5, 1)
    floor_log2 = k.astype(np.int64) - 1
    step_exp = np.where(a < MIN_NORMAL, SUBNORMAL_STEP_EXP, floor_log2 - 3)
    n = np.rint(np.ldexp(a, -step_exp))  # rint: round half to even
    y = np.ldexp(n, step_exp)  # the rounded magnitude, an E4M3 value

    # Bit fields of y (recomputed: rounding may carry into the next binade).
    _, ky = np.frexp(y)
    ey = ky.astype(np.int64) - 1
    sub = y < MIN_NORMAL
    exp_field = np.where(sub, 0, ey + 7)
    mant_sub = np.ldexp(y, -SUBNORMAL_STEP_EXP)
    mant_norm = np.ldexp(y, -ey) * 8.0 - 8.0
    mant = np.where(sub, mant_sub, mant_norm).astype(np.int64)
    code = (exp_field << 3) | mant | (neg.astype(np.int64) << 7)
    code = np.where(nan, 0x7F | (neg.astype(np.int64) << 7), code)
    return code.astype(np.uint8)


def finite_codes() -> np.ndarray:
    """The 254 non-NaN codes."""
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]
