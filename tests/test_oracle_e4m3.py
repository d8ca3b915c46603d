"""Pins for the oracle's E4M3 codec, against sources other than the oracle itself.

* torch's float8_e4m3fn type (a library implementation of OCP E4M3FN) for the
  decode table and for rounding of values up to 448;
* a brute-force nearest-value search (ties to the even code) over the library's
  table of values;
* textbook facts of the format (bias 7, 3 mantissa bits, max 448, min subnormal
  2^-9) and the widths the pages state.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3


def torch_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_widths_match_pages(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "pages_facts.json")))["e4m3"]
    # 1 sign + exponent + mantissa = 8 bits; the decode of code 0x08 is the
    # smallest normal 2^(1-bias) with bias 2^(e-1)-1.
    assert 1 + facts["exponent_bits"] + facts["mantissa_bits"] == 8
    bias = 2 ** (facts["exponent_bits"] - 1) - 1
    assert e4m3.decode(np.array([1 << facts["mantissa_bits"]]))[0] == 2.0 ** (1 - bias)
    # 2^mantissa_bits subnormal steps below the smallest normal
    assert e4m3.decode(np.array([1]))[0] == 2.0 ** (1 - bias - facts["mantissa_bits"])


def test_decode_matches_library_all_256():
    ours = e4m3.decode(np.arange(256))
    lib = torch_table()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))  # -0 at 0x80


def test_decode_textbook_values():
    d = e4m3.decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x80, 0x3C]))
    assert list(d[:7]) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -448.0]
    assert d[7] == 0.0 and np.signbit(d[7])
    assert d[8] == 1.5


def test_round_trip_254_finite_codes():
    c = e4m3.finite_codes()
    assert c.size == 254
    assert np.array_equal(e4m3.encode(e4m3.decode(c)), c)


def brute_force_encode(v):
    """Nearest non-negative library value to |v| (clamped to 448), ties to even code."""
    table = torch_table()[:0x7F]  # codes 0x00..0x7E, non-negative, finite
    out = np.empty(v.shape, dtype=np.uint8)
    for i, x in enumerate(v):
        a = min(abs(x), 448.0)
        d = np.abs(table - a)
        best = np.flatnonzero(d == d.min())
        if best.size > 1:
            best = best[(best & 1) == 0]
        assert best.size == 1
        out[i] = best[0] | (0x80 if np.signbit(x) else 0)
    return out


def test_encode_brute_force_midpoints():
    vals = torch_table()[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2  # exact in float64
    eps = np.spacing(mids)
    pts = np.concatenate([mids, mids + eps, mids - eps, vals])
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(e4m3.encode(pts), brute_force_encode(pts))
    # exact midpoints go to the even code, never the odd one
    assert np.all(e4m3.encode(mids) & 1 == 0)


def test_encode_brute_force_random():
    rng = np.random.default_rng(123)
    mag = np.exp2(rng.uniform(-12, 9.2, 4000))
    v = mag * rng.choice([-1.0, 1.0], mag.size)
    assert np.array_equal(e4m3.encode(v), brute_force_encode(v))


def test_encode_matches_library_up_to_448():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), 200000)).astype(np.float32)
    v = mag * rng.choice(np.array([-1, 1], np.float32), mag.size)
    vals = torch_table()[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in float32
    v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(v.astype(np.float64)), lib)


def test_saturation_and_zero_sign():
    v = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e9, np.inf, -500.0, -np.inf])
    assert list(e4m3.encode(v)) == [0x7E] * 7 + [0xFE] * 2
    z = e4m3.encode(np.array([0.0, -0.0, -1e-30, 1e-30, -2.0 ** -10]))
    assert list(z) == [0x00, 0x80, 0x80, 0x00, 0x80]


def test_underflow_boundary():
    # 2^-10 is halfway between 0 and the smallest subnormal 2^-9: ties to 0 (even)
    v = np.array([2.0 ** -10, 1.5 * 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -10 * (1 + 2.0 ** -30)])
    assert list(e4m3.encode(v)) == [0x00, 0x01, 0x02, 0x01]


def test_nan_propagates():
    c = e4m3.encode(np.array([np.nan, -np.nan]))
    assert (c[0] & 0x7F) == 0x7F and (c[1] & 0x7F) == 0x7F


@pytest.mark.parametrize("bit", range(8))
def test_single_bit_codes(bit):
    """Each code bit has the value the format's field layout gives it."""
    c = np.array([1 << bit], dtype=np.uint8)
    v = e4m3.decode(c)[0]
    if bit < 3:
        assert v == (1 << bit) * 2.0 ** -9  # mantissa bits of a subnormal
    elif bit < 7:
        assert v == 2.0 ** ((1 << (bit - 3)) - 7)  # exponent field 2^(bit-3)
    else:
        assert v == 0.0 and np.signbit(v)
