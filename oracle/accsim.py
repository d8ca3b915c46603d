"""Limited-precision accumulation model, for the K = 4096 demonstration.

"Six Reasons Deepseek Ai Is A Waste Of Time" (myomija.com) reports a
preliminary test in which the limited accumulation precision of Tensor Cores
gives a maximum relative error of nearly 2% for an FP8 GEMM with inner
dimension 4096 (the number is the only operand left of a sentence whose start
was lost from the page text), and the passage on promotion says MMA partials are
kept at limited bit width until they are copied to FP32 registers. The pages
state neither the accumulator's width nor the data nor the error metric. The
reading used here:

* Accumulator model. The K products, in K order, are accumulated in chunks of
  ``chunk`` terms. For each chunk, the running sum and the chunk's products are
  aligned to the largest exponent among them; every term is rounded (to nearest
  even, or toward zero) to ``mant_bits`` significant bits at that exponent; the
  rounded terms are added exactly and become the new running sum.
* Products are the exact products of the dequantized operands (code times scale),
  so the measured error is accumulation error only.
* Metric: the largest |C - C_ref| / |C_ref| over outputs with
  |C_ref| >= 0.1 * RMS(C_ref). Outputs that cancel to near zero are left out;
  on them any finite-precision sum has unbounded relative error.
* Per-group FP32 promotion, for comparison: each 128-term group of code products
  is summed in binary32 (products of two E4M3 codes are exact in binary32), then
  scaled by fl32(sa * sb) and added into a binary32 accumulator.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

from . import e4m3

GROUP = 128


def limited_sum(terms: np.ndarray, mant_bits: int = 14, chunk: int = 32,
                mode: str = "rne") -> np.ndarray:
    """Sum each row of ``terms`` (R x K, float64) with the chunked limited model."""
    terms = np.asarray(terms, dtype=np.float64)
    R, K = terms.shape
    acc = np.zeros(R, dtype=np.float64)
    for c0 in range(0, K, chunk):
        block = np.concatenate([acc[:, None], terms[:, c0:c0 + chunk]], axis=1)
        amax = np.max(np.abs(block), axis=1)
        _, k = np.frexp(amax)  # amax = f * 2^k, f in [0.5, 1)
        quantum_exp = (k.astype(np.int64) - 1) - (mant_bits - 1)
        scaled = np.ldexp(block, -quantum_exp[:, None])
        if mode == "rne":
            r = np.rint(scaled)
        elif mode == "rz":
            r = np.trunc(scaled)
        else:
            raise ValueError(mode)
        acc = np.where(amax > 0, np.ldexp(r.sum(axis=1), quantum_exp), 0.0)
    return acc


def _dequant_rows(codes, scales):
    R, K = codes.shape
    v = e4m3.decode(codes).reshape(R, K // GROUP, GROUP)
    return (v * np.asarray(scales, dtype=np.float64)[:, :, None]).reshape(R, K)


def products(qa, sa, qb, sb_rows):
    """Exact-order product tensor T[m, n, k] of the dequantized operands.

    sb_rows: the weight scale of each B row, shape N x K/128 (sb repeated per
    128-row block).
    """
    a = _dequant_rows(qa, sa)
    b = _dequant_rows(qb, sb_rows)
    return a[:, None, :] * b[None, :, :]


def per_group_fp32(qa, sa, qb, sb_rows) -> np.ndarray:
    """binary32 model of per-group promotion (see module docstring)."""
    M, K = qa.shape
    N = qb.shape[0]
    a = e4m3.decode(qa).astype(np.float32)
    b = e4m3.decode(qb).astype(np.float32)
    acc = np.zeros((M, N), dtype=np.float32)
    for g in range(K // GROUP):
        p = np.zeros((M, N), dtype=np.float32)
        for k in range(g * GROUP, (g + 1) * GROUP):
            p = (p + a[:, k][:, None] * b[:, k][None, :]).astype(np.float32)
        scale = (np.asarray(sa[:, g], np.float32)[:, None]
                 * np.asarray(sb_rows[:, g], np.float32)[None, :]).astype(np.float32)
        acc = (acc + (scale * p).astype(np.float32)).astype(np.float32)
    return acc


def max_rel_error(c, c_ref, floor_frac: float = 0.1) -> float:
    c = np.asarray(c, dtype=np.float64).ravel()
    c_ref = np.asarray(c_ref, dtype=np.float64).ravel()
    rms = np.sqrt(np.mean(c_ref ** 2))
    keep = np.abs(c_ref) >= floor_frac * rms
    return float(np.max(np.abs(c[keep] - c_ref[keep]) / np.abs(c_ref[keep])))


def demonstration(qa, sa, qb, sb_rows, mant_bits=14, chunk=32, mode="rne"):
    """Relative errors of the limited model and of per-group FP32 on one sample.

    Returns (limited_error, per_group_fp32_error, reference float64 outputs).
    """
    t = products(qa, sa, qb, sb_rows)
    M, N, K = t.shape
    flat = t.reshape(M * N, K)
    c_ref = flat.sum(axis=1)  # float64; its error is ~1e-16 relative
    c_lim = limited_sum(flat, mant_bits=mant_bits, chunk=chunk, mode=mode)
    c_pg = per_group_fp32(qa, sa, qb, sb_rows).ravel()
    return (max_rel_error(c_lim, c_ref), max_rel_error(c_pg, c_ref),
            c_ref.reshape(M, N))
