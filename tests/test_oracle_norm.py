"""Pins for the oracle's normalization + 1x128 cast (oracle/norm.py).

Independent references: torch's float64 rms_norm / layer_norm (library
routines), closed forms for constant power-of-two rows, power-of-two
invariance, exact rational sums for the statistics, the normalized moments,
and torch's binary32 division + float8_e4m3fn cast for the final quantization.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_fine_grained_online_amd import synthetic as S
from oracle import bf16, norm, quant


def bits(v):
    return S.f32_to_bf16_bits(np.asarray(v, np.float32))


def ulp32(v):
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.maximum(v, 2.0 ** -126))
    return np.ldexp(1.0, e - 24)


def inputs(M, K, seed):
    x = S.activations(M, K, S.rng_for(seed, 0))
    g = bits(1.0 + 0.1 * S.rng_for(seed, 1).standard_normal(K))
    b = bits(0.05 * S.rng_for(seed, 2).standard_normal(K))
    return x, g, b


def test_rms_norm_matches_torch_float64():
    x, g, _ = inputs(64, 1024, 970)
    # an eps large enough that dropping it would fail the comparison
    y = norm.rms_norm_f32(x, g, 0.25)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(bf16.to_f64(x)), (1024,),
                                       torch.from_numpy(bf16.to_f64(g)), eps=0.25).numpy()
    assert y.dtype == np.float32
    assert np.all(np.abs(y - ref) <= 4 * ulp32(ref))


def test_layer_norm_matches_torch_float64():
    x, g, b = inputs(64, 1024, 971)
    y = norm.layer_norm_f32(x, g, b, 0.25)
    x64 = bf16.to_f64(x)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x64), (1024,),
                                         torch.from_numpy(bf16.to_f64(g)),
                                         torch.from_numpy(bf16.to_f64(b)), eps=0.25).numpy()
    mu = x64.mean(axis=1, keepdims=True)
    r = 1 / np.sqrt(x64.var(axis=1, keepdims=True) + 0.25)
    # rounding of mu to binary32 perturbs x - mu by up to ulp(mu)/2; the three
    # binary32 roundings before "+ beta" are relative to |gamma (x - mu) r|,
    # which can be far larger than the result when beta cancels it
    g64 = np.abs(bf16.to_f64(g))
    tol = (2 * ulp32(ref) + g64 * r * (ulp32(mu) / 2 + ulp32(x64 - mu))
           + 4 * 2.0 ** -24 * g64 * np.abs(x64 - mu) * r)
    assert np.all(np.abs(y - ref) <= tol)


@pytest.mark.parametrize("j", [-30, -3, 0, 7, 40])
def test_constant_power_of_two_rows_give_gamma(j):
    """x = +-2^j in every position, eps = 0: r = 2^-j exactly and y = +-gamma."""
    K = 256
    x = np.tile(bits([2.0 ** j, -(2.0 ** j)])[:, None], (1, K))
    g = bits(np.linspace(-3, 3, K))
    y = norm.rms_norm_f32(x, g, 0.0)
    assert np.array_equal(y[0], bf16.to_f32(g)) and np.array_equal(y[1], -bf16.to_f32(g))


@pytest.mark.parametrize("j", [-12, 5])
def test_power_of_two_invariance(j):
    x, g, b = inputs(16, 512, 972)
    xs = bits(np.ldexp(bf16.to_f32(x), j))
    assert np.array_equal(norm.rms_norm_f32(x, g, 0.0), norm.rms_norm_f32(xs, g, 0.0))
    assert np.array_equal(norm.layer_norm_f32(x, g, b, 0.0), norm.layer_norm_f32(xs, g, b, 0.0))
    assert all(np.array_equal(u, v) for u, v in zip(norm.norm_quant_act_1x128(x, g, 0.0),
                                                       norm.norm_quant_act_1x128(xs, g, 0.0)))


def test_statistics_are_exact_sums():
    """A row whose naive float64 sum loses the small terms: 2^60, then ones,
    then -2^60. The mean (and so the centring) must see the ones."""
    K = 128
    row = np.ones(K)
    row[0], row[-1] = 2.0 ** 60, -(2.0 ** 60)
    x = bits(row)[None, :]
    exact = Fraction(K - 2, K)
    assert norm._exact_row_sums(bf16.to_f64(x))[0] / K == float(exact)
    naive = 0.0
    for v in bf16.to_f64(x)[0]:
        naive += v
    assert naive != float(K - 2)  # the plain left-to-right float64 sum would be wrong
    sq = norm._exact_row_sums(bf16.to_f64(x) ** 2)[0]
    assert sq == float(2 * Fraction(2) ** 120 + (K - 2))


def test_layer_norm_output_moments():
    """With gamma = 1, beta = 0 every row has mean ~0 and variance ~1."""
    x, _, _ = inputs(32, 2048, 973)
    K = 2048
    y = norm.layer_norm_f32(x, bits(np.ones(K)), bits(np.zeros(K)), 0.0).astype(np.float64)
    assert np.all(np.abs(y.mean(axis=1)) < 1e-5)
    assert np.all(np.abs(y.var(axis=1) - 1) < 1e-5)


def test_quantization_of_normalized_rows_matches_library_cast():
    x, g, b = inputs(64, 512, 974)
    for centred in (False, True):
        q, s = norm.norm_quant_act_1x128(x, g, 1e-6, b, centred)
        y = norm.layer_norm_f32(x, g, b, 1e-6) if centred else norm.rms_norm_f32(x, g, 1e-6)
        yt = torch.from_numpy(y).reshape(64, 4, 128)
        st = yt.abs().amax(dim=2, keepdim=True) / 448.0
        qt = (yt / st).to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 512).numpy()
        assert np.array_equal(q, qt)
        assert np.array_equal(s, st.reshape(64, 4).numpy())
        assert np.all(np.any((q.reshape(64, 4, 128) & 0x7F) == 0x7E, axis=2))


def test_zero_row_normalizes_to_beta():
    K = 256
    x = np.zeros((1, K), np.uint16)
    g = bits(np.full(K, 2.0))
    b = bits(np.linspace(-1, 1, K))
    assert np.all(norm.rms_norm_f32(x, g, 1e-6) == 0)
    assert np.array_equal(norm.layer_norm_f32(x, g, b, 1e-6)[0], bf16.to_f32(b))
    q, s = quant.quant_act_1x128(x)
    assert np.array_equal(norm.norm_quant_act_1x128(x, g, 1e-6)[0], q) and np.all(s == 0)
