"""Block-scaled FP8 GEMM, dense and grouped (MoE), as exact per-group sums.

What is computed, for A codes M x K with 1x128 scales sa[M][K/128] and B codes
N x K (out-channels x in-channels) with 128x128 scales sb[N/128][K/128]:

  P_g[m, n] = sum_{k in group g} dec(qa[m, k]) * dec(qb[n, k])     (exact)
  C[m, n]   = sum_g (sa[m, g] * sb[n // 128, g]) * P_g[m, n]         (float64)
  output    = C rounded once to float32, or once to bf16 (RNE)

P_g is exact in float64 for any summation order: each product of two E4M3
values is a multiple of 2^-18 below 448^2 < 2^18 in magnitude, so a 128-term
group sum is a multiple of 2^-18 below 2^25, which needs at most 43 of
float64's 53 significand bits. A float64 matrix product per group is therefore
exactly the naive triple loop. The scale product of two binary32 values is
exact in float64; the rest adds at most a few float64 roundings, far below
binary32 resolution.

Sources:
* "Six Reasons Deepseek Ai Is A Waste Of Time" (myomija.com): the GEMMs take
  FP8 tensors and produce BF16 or FP32 (paragraph on the GEMM operands); the
  per-group scaling factors along K are multiplied in during dequantization
  (paragraph on fine-grained quantization); MMA partials are promoted to FP32
  registers at an interval and accumulated there at full precision (passage on
  promotion). The interval's symbol was lost from the page text; the reading
  used is one 128-wide K group, the span of one scaling factor.
* Japanese codingmall.com page, item 8: the GEMM library covers dense and MoE
  (grouped) layers. Grouped reading: expert e owns rows
  [m_offsets[e], m_offsets[e+1]) of A and of C and uses its own B_e, sb_e.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

from . import bf16, e4m3

GROUP = 128


def _check(qa, sa, qb, sb):
    M, K = qa.shape
    N, K2 = qb.shape
    if K != K2 or K % GROUP or N % GROUP:
        raise ValueError("shape mismatch: need A MxK, B NxK, K%128==0, N%128==0")
    if sa.shape != (M, K // GROUP) or sb.shape != (N // GROUP, K // GROUP):
        raise ValueError("scale shape mismatch")
    return M, N, K


def gemm_blockscaled_f64(qa, sa, qb, sb) -> np.ndarray:
    """C (float64, M x N) before the final rounding."""
    M, N, K = _check(qa, sa, qb, sb)
    a = e4m3.decode(qa)
    b = e4m3.decode(qb)
    sa64 = np.asarray(sa, dtype=np.float64)
    sb64 = np.asarray(sb, dtype=np.float64)
    c = np.zeros((M, N), dtype=np.float64)
    for g in range(K // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        p = a[:, ks] @ b[:, ks].T  # exact (see module docstring)
        scale = sa64[:, g][:, None] * np.repeat(sb64[:, g], GROUP)[None, :]
        c += scale * p
    return c


def abs_sum(qa, sa, qb, sb) -> np.ndarray:
    """S[m, n] = sum_k |a_k * sa| * |b_k * sb|: the scale of the FP32 tolerance."""
    M, N, K = _check(qa, sa, qb, sb)
    a = np.abs(e4m3.decode(qa))
    b = np.abs(e4m3.decode(qb))
    sa64 = np.abs(np.asarray(sa, dtype=np.float64))
    sb64 = np.abs(np.asarray(sb, dtype=np.float64))
    s = np.zeros((M, N), dtype=np.float64)
    for g in range(K // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        p = a[:, ks] @ b[:, ks].T
        s += sa64[:, g][:, None] * np.repeat(sb64[:, g], GROUP)[None, :] * p
    return s


def gemm_rowscaled_f64(qa, sa, qb, sb_rows) -> np.ndarray:
    """C = A * B^T with 1x128 scales on both operands (sb_rows: N x K/128).

    The weight-gradient GEMM: both operands are activations/gradients
    quantized per 1x128 tile along the reduction dimension, so the promotion
    scale of group g is sa[m, g] * sb_rows[n, g].
    """
    M, K = qa.shape
    N, K2 = qb.shape
    if K != K2 or K % GROUP:
        raise ValueError("shape mismatch: need A MxK, B NxK, K%128==0")
    if sa.shape != (M, K // GROUP) or sb_rows.shape != (N, K // GROUP):
        raise ValueError("scale shape mismatch")
    a = e4m3.decode(qa)
    b = e4m3.decode(qb)
    sa64 = np.asarray(sa, dtype=np.float64)
    sb64 = np.asarray(sb_rows, dtype=np.float64)
    c = np.zeros((M, N), dtype=np.float64)
    for g in range(K // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        c += (sa64[:, g][:, None] * sb64[:, g][None, :]) * (a[:, ks] @ b[:, ks].T)
    return c


def abs_sum_rowscaled(qa, sa, qb, sb_rows) -> np.ndarray:
    M, K = qa.shape
    a = np.abs(e4m3.decode(qa))
    b = np.abs(e4m3.decode(qb))
    s = np.zeros((M, qb.shape[0]), dtype=np.float64)
    for g in range(K // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        s += (np.abs(np.asarray(sa[:, g], np.float64))[:, None]
              * np.abs(np.asarray(sb_rows[:, g], np.float64))[None, :]) * (a[:, ks] @ b[:, ks].T)
    return s


def round_f32(c64: np.ndarray) -> np.ndarray:
    return np.asarray(c64, dtype=np.float64).astype(np.float32)


def round_bf16(c64: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16), rounded once from float64."""
    return bf16.round_from_f64(c64)


def gemm_blockscaled(qa, sa, qb, sb, out: str = "f32"):
    c64 = gemm_blockscaled_f64(qa, sa, qb, sb)
    if out == "f32":
        return round_f32(c64)
    if out == "bf16":
        return round_bf16(c64)
    raise ValueError(out)


def check_offsets(m_offsets, G: int, M_total: int):
    off = np.asarray(m_offsets, dtype=np.int64)
    if off.shape != (G + 1,) or off[0] != 0 or off[-1] != M_total:
        raise ValueError("m_offsets must have G+1 entries from 0 to M_total")
    if np.any(np.diff(off) < 0) or np.any(off % GROUP):
        raise ValueError("m_offsets must be nondecreasing multiples of 128")
    return off


def gemm_grouped_f64(qa, sa, qb, sb, m_offsets) -> np.ndarray:
    """qb: G x N x K codes, sb: G x N/128 x K/128. Rows of expert e use B_e."""
    qb = np.asarray(qb)
    G, N, K = qb.shape
    M = qa.shape[0]
    off = check_offsets(m_offsets, G, M)
    c = np.zeros((M, N), dtype=np.float64)
    for e in range(G):
        r = slice(int(off[e]), int(off[e + 1]))
        if off[e + 1] > off[e]:
            c[r] = gemm_blockscaled_f64(qa[r], sa[r], qb[e], sb[e])
    return c


def abs_sum_grouped(qa, sa, qb, sb, m_offsets) -> np.ndarray:
    qb = np.asarray(qb)
    G, N, K = qb.shape
    M = qa.shape[0]
    off = check_offsets(m_offsets, G, M)
    s = np.zeros((M, N), dtype=np.float64)
    for e in range(G):
        r = slice(int(off[e]), int(off[e + 1]))
        if off[e + 1] > off[e]:
            s[r] = abs_sum(qa[r], sa[r], qb[e], sb[e])
    return s


def expert_of_rows(m_offsets, rows) -> np.ndarray:
    """Expert index owning each row (for sampled checks at full size)."""
    off = np.asarray(m_offsets, dtype=np.int64)
    return np.searchsorted(off, np.asarray(rows), side="right") - 1
