"""Pins for the oracle's tolerance helpers, against references other than
themselves (CPU):

* gemm.abs_sum, abs_sum_rowscaled and abs_sum_grouped, the S in every FP32
  tolerance, against an exact rational (fractions.Fraction) brute force of
  sum_k |dec(a_k) sa| |dec(b_k) sb|, with negative codes and negative scales
  present (a dropped absolute value or a wrong scale index shows);
* bf16.ulp against the distance between adjacent bf16 values as torch decodes
  them (the spacing above each value);
* accsim.per_group_fp32 against closed forms fixed by IEEE binary32 rounding:
  a group sum that binary32 cannot hold, a scale product that rounds to even,
  and an accumulator whose result depends on adding the groups in K order.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import accsim, bf16, e4m3, gemm

TAB = [Fraction(float(v)) if not np.isnan(v) else None for v in e4m3.decode(np.arange(256))]


def finite_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    return c


def brute_S(qa, sa, qb, sb_rows):
    """Exact sum_k |a_k sa[m, k/128]| |b_k sb_rows[n, k/128]| as Fractions."""
    M, K = qa.shape
    N = qb.shape[0]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // 128
                acc += (abs(TAB[int(qa[m, k])] * Fraction(float(sa[m, g])))
                        * abs(TAB[int(qb[n, k])] * Fraction(float(sb_rows[n, g]))))
            out[m, n] = acc
    return out


def assert_close(got, exact, rel=2.0 ** -50):
    for (m, n), ex in np.ndenumerate(exact):
        assert abs(Fraction(float(got[m, n])) - ex) <= rel * ex, (m, n)


@pytest.mark.parametrize("M,N,K,seed", [(2, 128, 256, 0), (3, 256, 128, 1)])
def test_abs_sum_against_fraction_brute_force(M, N, K, seed):
    rng = np.random.default_rng(seed)
    qa, qb = finite_codes(rng, (M, K)), finite_codes(rng, (N, K))
    sa = (rng.uniform(0.1, 3, (M, K // 128)) * rng.choice([-1, 1], (M, K // 128))).astype(np.float32)
    sb = (rng.uniform(0.1, 3, (N // 128, K // 128)) * rng.choice([-1, 1], (N // 128, K // 128))).astype(np.float32)
    n_cols = [0, 1, 127, N - 1]  # brute force on a few columns (both weight blocks when N = 256)
    got = gemm.abs_sum(qa, sa, qb, sb)[:, n_cols]
    exact = brute_S(qa, sa, qb[n_cols], np.repeat(sb, 128, axis=0)[n_cols])
    assert_close(got, exact)


def test_abs_sum_rowscaled_against_fraction_brute_force():
    rng = np.random.default_rng(5)
    M, N, K = 3, 5, 256
    qa, qb = finite_codes(rng, (M, K)), finite_codes(rng, (N, K))
    sa = (rng.uniform(0.1, 3, (M, 2)) * rng.choice([-1, 1], (M, 2))).astype(np.float32)
    sbr = (rng.uniform(0.1, 3, (N, 2)) * rng.choice([-1, 1], (N, 2))).astype(np.float32)
    assert_close(gemm.abs_sum_rowscaled(qa, sa, qb, sbr), brute_S(qa, sa, qb, sbr))


def test_abs_sum_grouped_against_fraction_brute_force():
    rng = np.random.default_rng(6)
    G, N, K = 3, 128, 128
    off = np.array([0, 128, 128, 256], np.int32)  # expert 1 is empty
    qa = finite_codes(rng, (256, K))
    sa = rng.uniform(0.1, 3, (256, 1)).astype(np.float32)
    qb = finite_codes(rng, (G, N, K))
    sb = rng.uniform(0.1, 3, (G, 1, 1)).astype(np.float32)
    got = gemm.abs_sum_grouped(qa, sa, qb, sb, off)
    rows, cols = [0, 127, 128, 255], [0, 77]
    for r in rows:
        e = 0 if r < 128 else 2
        ex = brute_S(qa[[r]], sa[[r]], qb[e][cols], np.repeat(sb[e], 128, axis=0)[cols])
        assert_close(got[[r]][:, cols], ex)


def test_bf16_ulp_is_the_spacing_to_the_next_value():
    """For every finite positive bf16 value below the largest, ulp() equals the
    distance to the next bf16 value up, both decoded by torch; ulp is symmetric
    in the sign and is the subnormal spacing at zero."""
    bits = np.arange(0x0000, 0x7F7F, dtype=np.uint16)  # 0 .. next-to-largest finite
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nxt = torch.from_numpy((bits + 1).view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16.ulp(bits), nxt - vals)
    assert np.array_equal(bf16.ulp(bits | 0x8000), bf16.ulp(bits))
    assert bf16.ulp(np.array([0], np.uint16))[0] == 2.0 ** -133


def _codes(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_per_group_fp32_group_sum_is_binary32():
    """One group: 448 * 448 = 200704 then 127 products 2^-9 * 2^-9 = 2^-18. In
    binary32 at 200704 (spacing 2^-6) each small product is below half a
    spacing and is lost: the group sum is 200704, where float64 would keep
    200704 + 127 * 2^-18."""
    qa = _codes([[448.0] + [2.0 ** -9] * 127])
    qb = _codes([[448.0] + [2.0 ** -9] * 127])
    one = np.ones((1, 1), np.float32)
    assert accsim.per_group_fp32(qa, one, qb, one)[0, 0] == np.float32(200704.0)
    exact = gemm.gemm_rowscaled_f64(qa, one, qb, one)[0, 0]
    assert exact == 200704.0 + 127 * 2.0 ** -18


def test_per_group_fp32_scale_product_rounds_to_even():
    """sa = sb = 1 + 2^-12: sa * sb = 1 + 2^-11 + 2^-24 is a binary32 tie and
    rounds to the even 1 + 2^-11; with P = 1 the output is exactly that."""
    qa = _codes([[1.0] + [0.0] * 127])
    qb = _codes([[1.0] + [0.0] * 127])
    s = np.array([[1 + 2.0 ** -12]], np.float32)
    assert accsim.per_group_fp32(qa, s, qb, s)[0, 0] == np.float32(1 + 2.0 ** -11)


def test_per_group_fp32_adds_groups_in_k_order():
    """Groups contribute 1, 2^-24, 2^-24 (2^-6 * 2^-6 = 2^-12 times a scale of
    2^-12). In K order each 1 + 2^-24 is a tie that rounds back to 1, so the
    result is 1; in reverse order the two small terms make 2^-23 first and the
    result is 1 + 2^-23."""
    K = 384
    a = np.zeros((1, K), np.float32)
    b = np.zeros((1, K), np.float32)
    a[0, 0], b[0, 0] = 1.0, 1.0
    a[0, 128], b[0, 128] = 2.0 ** -6, 2.0 ** -6
    a[0, 256], b[0, 256] = 2.0 ** -6, 2.0 ** -6
    sa = np.array([[1.0, 2.0 ** -12, 2.0 ** -12]], np.float32)
    sb = np.ones((1, 3), np.float32)
    assert accsim.per_group_fp32(_codes(a), sa, _codes(b), sb)[0, 0] == np.float32(1.0)
    rev = accsim.per_group_fp32(_codes(a[:, ::-1].copy()), sa[:, ::-1].copy(),
                                _codes(b[:, ::-1].copy()), sb)[0, 0]
    assert rev == np.float32(1 + 2.0 ** -23)
