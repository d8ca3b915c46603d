"""Pins for the oracle's 1x128 / 128x128 quantization.

Independent references used:
* torch (library): binary32 division and the float8_e4m3fn cast, over the
  exhaustive table of (amax significand, x) pairs at several amax exponents;
* exact rational arithmetic (fractions.Fraction) with a brute-force nearest
  search, on small tiles;
* invariants the definition implies: power-of-two invariance of the codes, the
  amax element mapping to +-448, locality (online: a tile's codes depend on that
  tile only), the RNE error bound, and the relation between the two
  granularities.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_fine_grained_online_amd import synthetic as S
from oracle import bf16, e4m3, quant


def torch_quant_tiles(x_bits):
    """Library reference: s = fl32(amax/448), q = float8_e4m3fn(fl32(x/s))."""
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float()
    M, K = x.shape
    xt = x.reshape(M, K // 128, 128)
    amax = xt.abs().amax(dim=2, keepdim=True)
    s = amax / 448.0
    q = torch.where(s == 0, xt, xt / s)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(M, K)
    return codes.numpy(), s.reshape(M, K // 128).numpy()


@pytest.mark.parametrize("exp_field", [127, 1, 0, 30, 60, 64, 200, 254])
def test_exhaustive_table_vs_library(exp_field):
    tiles = S.exhaustive_tiles(exp_field)
    codes, s = quant.quant_act_1x128(tiles)
    lib_codes, lib_s = torch_quant_tiles(tiles)
    assert np.array_equal(s.view(np.uint32), lib_s.view(np.uint32))
    assert np.array_equal(codes, lib_codes)


def test_tile_size_matches_pages(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "pages_facts.json")))
    assert (facts["activation_tile"]["rows"], facts["activation_tile"]["cols"]) == (1, quant.GROUP)
    assert (facts["weight_block"]["rows"], facts["weight_block"]["cols"]) == (quant.GROUP, quant.GROUP)


def _fraction_round_f32(q: Fraction) -> Fraction:
    """Exact rational -> nearest binary32 value (ties to even), by brute force."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (max(e, -126) - 23)
    n = a / step
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * step


def _brute_e4m3(v: Fraction, neg: bool) -> int:
    table = [Fraction(float(t)) for t in
             torch.arange(0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double()]
    a = min(abs(v), Fraction(448))
    d = [abs(t - a) for t in table]
    m = min(d)
    best = [i for i, di in enumerate(d) if di == m]
    if len(best) > 1:
        best = [i for i in best if i % 2 == 0]
    return best[0] | (0x80 if neg else 0)


def test_exact_rational_brute_force():
    rng = np.random.default_rng(5)
    x = S.activations(3, 256, rng)
    # include tiles with a bf16 subnormal and a huge amax
    x[2, :128] = (x[2, :128] & 0x807F)  # exponent field 0: subnormals
    x[2, 128:] = (x[2, 128:] & 0x80FF) | 0x7A00
    codes, s = quant.quant_act_1x128(x)
    xv = bf16.to_f32(x)
    for m in range(x.shape[0]):
        for g in range(2):
            tile = [Fraction(float(v)) for v in xv[m, g * 128:(g + 1) * 128]]
            amax = max(abs(t) for t in tile)
            s_exact = _fraction_round_f32(amax / 448)
            assert Fraction(float(s[m, g])) == s_exact
            for k in range(128):
                neg = bool(np.signbit(xv[m, g * 128 + k]))
                if s_exact == 0:
                    want = 0x80 if neg else 0
                else:
                    want = _brute_e4m3(_fraction_round_f32(tile[k] / s_exact), neg)
                assert codes[m, g * 128 + k] == want, (m, g, k)


def test_amax_maps_to_448_and_scale_definition():
    x = S.activations(64, 1024, S.rng_for(99, 0))
    codes, s = quant.quant_act_1x128(x)
    c = codes.reshape(64, 8, 128)
    assert np.all(np.any((c & 0x7F) == 0x7E, axis=2))
    xv = bf16.to_f32(x).reshape(64, 8, 128)
    amax = np.abs(xv).max(axis=2)
    # s is the dequantization factor: 448 * s reproduces amax within binary32 rounding
    assert np.allclose(448.0 * s.astype(np.float64), amax, rtol=2 ** -23, atol=0)


@pytest.mark.parametrize("j", [-20, -7, -1, 1, 3, 20])
def test_power_of_two_invariance(j):
    x = S.activations(16, 512, S.rng_for(98, 0))
    codes, s = quant.quant_act_1x128(x)
    xs = S.f32_to_bf16_bits(np.ldexp(bf16.to_f32(x), j).astype(np.float32))
    codes2, s2 = quant.quant_act_1x128(xs)
    assert np.array_equal(codes, codes2)
    assert np.array_equal(s2, np.ldexp(s, j).astype(np.float32))


def test_locality_online_scales():
    x = S.activations(8, 512, S.rng_for(97, 0))
    codes, s = quant.quant_act_1x128(x)
    y = x.copy()
    y[3, 128:256] = S.f32_to_bf16_bits(bf16.to_f32(y[3, 128:256]) * np.float32(1000.0))
    codes2, s2 = quant.quant_act_1x128(y)
    mask = np.ones_like(codes, bool)
    mask[3, 128:256] = False
    assert np.array_equal(codes[mask], codes2[mask])
    smask = np.ones_like(s, bool)
    smask[3, 1] = False
    assert np.array_equal(s[smask], s2[smask]) and s2[3, 1] != s[3, 1]


def test_error_bound():
    x = S.activations(32, 1024, S.rng_for(96, 0))
    codes, s = quant.quant_act_1x128(x)
    xv = bf16.to_f32(x).astype(np.float64).reshape(32, 8, 128)
    dq = quant.dequant_act(codes, s).reshape(32, 8, 128)
    s3 = s.astype(np.float64)[:, :, None]
    q = np.abs(xv / s3)
    _, k = np.frexp(np.maximum(q, 2.0 ** -6))
    half_ulp = np.ldexp(1.0, k - 1 - 3) / 2  # E4M3 spacing / 2 at |x/s|
    bound = s3 * (half_ulp + q * 2.0 ** -24)
    assert np.all(np.abs(dq - xv) <= bound)


def test_zero_tile():
    x = np.zeros((2, 256), np.uint16)
    x[1, :128] = 0x8000  # -0
    x[0, 128:] = S.f32_to_bf16_bits(np.linspace(-1, 1, 128, dtype=np.float32))
    codes, s = quant.quant_act_1x128(x)
    assert s[0, 0] == 0 and s[1, 0] == 0 and s[1, 1] == 0 and s[0, 1] > 0
    assert np.all(codes[0, :128] == 0x00) and np.all(codes[1, :128] == 0x80)
    assert np.all(codes[1, 128:] == 0x00)


def test_weight_block_equals_act_tiles_when_every_row_holds_block_max():
    rng = S.rng_for(95, 0)
    w = S.weights(256, 384, rng)
    wv = bf16.to_f32(w).reshape(2, 128, 3, 128)
    peak = np.float32(0.5)
    wv = np.clip(wv, -0.25, 0.25)
    wv[:, :, :, 7] = peak  # every 1x128 row of every block holds the block max
    w2 = S.f32_to_bf16_bits(wv.reshape(256, 384))
    cw, sw = quant.quant_weight_128x128(w2)
    ca, sa = quant.quant_act_1x128(w2)
    assert np.array_equal(cw, ca)
    assert np.array_equal(np.repeat(sw, 128, axis=0), sa)


def test_weight_block_scale_layout_brute_force():
    rng = S.rng_for(94, 0)
    w = S.weights(384, 256, rng)
    cw, sw = quant.quant_weight_128x128(w)
    wv = bf16.to_f32(w)
    assert sw.shape == (3, 2)
    for nb in range(3):
        for g in range(2):
            blk = wv[nb * 128:(nb + 1) * 128, g * 128:(g + 1) * 128]
            amax = max(abs(float(v)) for v in blk.ravel())
            assert sw[nb, g] == np.float32(np.float32(amax) / np.float32(448.0))
    # every block has an element coded +-448
    c = cw.reshape(3, 128, 2, 128)
    assert np.all(np.any((c & 0x7F) == 0x7E, axis=(1, 3)))
