"""Pins for the oracle's block-scaled GEMM (dense and grouped) and bf16 rounding.

Independent references used:
* exact rational triple loops (fractions.Fraction) on tiny shapes;
* one-hot operands, which isolate every index (row, column, K group, scale);
* the special case where every scale is exactly 1, which reduces the GEMM to a
  plain float64 matrix product (library routine);
* separability over K groups and the grouped = concatenated-dense identity;
* torch's float32 -> bfloat16 cast and closed-form midpoints for bf16 rounding.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_fine_grained_online_amd import synthetic as S
from oracle import bf16, e4m3, gemm, quant


def small_operands(M, N, K, seed):
    a = S.activations(M, K, S.rng_for(900 + seed, 0))
    b = S.weights(N, K, S.rng_for(900 + seed, 1))
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    return qa, sa, qb, sb


def fraction_gemm(qa, sa, qb, sb):
    M, K = qa.shape
    N = qb.shape[0]
    tab = [Fraction(float(v)) if not np.isnan(v) else None for v in e4m3.decode(np.arange(256))]
    A = [[tab[int(c)] for c in row] for row in qa]
    B = [[tab[int(c)] for c in row] for row in qb]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // 128
                acc += A[m][k] * B[n][k] * Fraction(float(sa[m, g])) * Fraction(float(sb[n // 128, g]))
            out[m][n] = acc
    return out


@pytest.mark.parametrize("M,N,K,seed", [(3, 128, 128, 0), (2, 256, 256, 1), (2, 128, 384, 2)])
def test_exact_rational_tiny(M, N, K, seed):
    qa, sa, qb, sb = small_operands(M, N, K, seed)
    c64 = gemm.gemm_blockscaled_f64(qa, sa, qb, sb)
    exact = fraction_gemm(qa, sa, qb, sb)
    S_ = gemm.abs_sum(qa, sa, qb, sb)
    c32 = gemm.round_f32(c64)
    cb = gemm.round_bf16(c64)
    for m in range(M):
        for n in range(N):
            ex = exact[m][n]
            assert abs(Fraction(float(c64[m, n])) - ex) <= Fraction(2) ** -48 * Fraction(float(S_[m, n]))
            assert c32[m, n] == np.float32(float(ex))  # RN of the exact value
            assert cb[m, n] == bf16.round_from_f64(np.array([float(ex)]))[0]


def test_one_hot_indexing():
    M, N, K = 40, 384, 512
    rng = np.random.default_rng(3)
    sa = rng.uniform(0.5, 2.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, (N // 128, K // 128)).astype(np.float32)
    for m0, n0, k0 in [(0, 0, 0), (17, 129, 127), (39, 383, 128), (5, 255, 511), (31, 128, 300)]:
        qa = np.zeros((M, K), np.uint8)
        qb = np.zeros((N, K), np.uint8)
        qa[m0, k0] = 0x3C  # 1.5
        qb[n0, k0] = 0xC4  # -3.0
        c = gemm.gemm_blockscaled_f64(qa, sa, qb, sb)
        want = 1.5 * -3.0 * float(sa[m0, k0 // 128]) * float(sb[n0 // 128, k0 // 128])
        assert c[m0, n0] == want
        c[m0, n0] = 0
        assert not np.any(c)


def test_unit_scales_reduce_to_plain_matmul():
    """Every tile/block holds 448 and only E4M3 values -> all scales 1 -> C = A @ B^T."""
    rng = np.random.default_rng(4)
    M, N, K = 64, 256, 384
    finite = e4m3.decode(e4m3.finite_codes())
    a = rng.choice(finite, (M, K))
    b = rng.choice(finite, (N, K))
    a[:, ::128] = 448.0  # one 448 in every 1x128 tile
    b[::128, ::128] = -448.0  # one in every 128x128 block
    a_bits = S.f32_to_bf16_bits(a.astype(np.float32))
    b_bits = S.f32_to_bf16_bits(b.astype(np.float32))
    qa, sa = quant.quant_act_1x128(a_bits)
    qb, sb = quant.quant_weight_128x128(b_bits)
    assert np.all(sa == 1.0) and np.all(sb == 1.0)
    c = gemm.gemm_blockscaled_f64(qa, sa, qb, sb)
    assert np.array_equal(c, a @ b.T)


def test_group_separability():
    qa, sa, qb, sb = small_operands(48, 256, 512, 5)
    c = gemm.gemm_blockscaled_f64(qa, sa, qb, sb)
    parts = sum(gemm.gemm_blockscaled_f64(qa[:, g * 128:(g + 1) * 128], sa[:, g:g + 1],
                                          qb[:, g * 128:(g + 1) * 128], sb[:, g:g + 1])
                for g in range(4))
    S_ = gemm.abs_sum(qa, sa, qb, sb)
    assert np.all(np.abs(c - parts) <= 2.0 ** -50 * S_)


def test_grouped_is_concatenation_of_dense():
    rng = np.random.default_rng(6)
    G, N, K = 5, 256, 256
    off = np.array([0, 128, 128, 384, 512, 640], np.int32)  # expert 1 empty
    a = S.activations(int(off[-1]), K, S.rng_for(910, 0))
    a[120:128] = 0  # padding rows inside expert 0
    b = np.stack([S.weights(N, K, S.rng_for(910, 1 + e)) for e in range(G)])
    qa, sa = quant.quant_act_1x128(a)
    q = [quant.quant_weight_128x128(b[e]) for e in range(G)]
    qb = np.stack([x[0] for x in q])
    sb = np.stack([x[1] for x in q])
    c = gemm.gemm_grouped_f64(qa, sa, qb, sb, off)
    for e in range(G):
        r = slice(off[e], off[e + 1])
        if off[e + 1] > off[e]:
            assert np.array_equal(c[r], gemm.gemm_blockscaled_f64(qa[r], sa[r], qb[e], sb[e]))
    assert not np.any(c[120:128])  # zero padding rows give zero outputs
    assert list(gemm.expert_of_rows(off, [0, 127, 128, 383, 384, 639])) == [0, 0, 2, 2, 3, 4]
    with pytest.raises(ValueError):
        gemm.check_offsets([0, 100, 256], 2, 256)


def test_bf16_rounding_vs_library_on_float32_values():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(100000) * np.exp2(rng.uniform(-130, 120, 100000))).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.round_from_f64(v.astype(np.float64)), lib)


def test_bf16_rounding_midpoints_float64():
    vals = bf16.to_f64(np.arange(0x3F00, 0x3F80, dtype=np.uint16))  # [0.5, 1)
    mids = (vals[:-1] + vals[1:]) / 2
    up = bf16.round_from_f64(mids + 2.0 ** -40)
    down = bf16.round_from_f64(mids - 2.0 ** -40)
    tie = bf16.round_from_f64(mids)
    lo = np.arange(0x3F00, 0x3F7F, dtype=np.uint16)
    assert np.array_equal(down, lo) and np.array_equal(up, lo + 1)
    assert np.all(tie & 1 == 0)
    # float64 value just above a float32 midpoint of bf16: no double rounding
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert bf16.round_from_f64(np.array([x]))[0] == 0x3F81
    assert bf16.round_from_f64(np.array([3.5e38, -3.5e38, 3.0e38])).tolist() == [0x7F80, 0xFF80, 0x7F62]
