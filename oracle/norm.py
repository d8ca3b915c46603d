"""Layer normalization fused with the 1x128 FP8 cast.

The woojincopolymer.co.kr post (the paragraph of hardware suggestions) asks for
a warp-level cast instruction so that layer normalization and the FP8 cast can
be fused; "Six Reasons Deepseek Ai Is A Waste Of Time" keeps normalization
operators in higher precision (BF16 or FP32) while the GEMMs run in FP8. The
plain reading: the normalization runs in higher precision, and its output goes
straight into the 1x128 activation quantizer, without a BF16 copy in between.

What is computed, per row x (K bf16 values, exact in float64):

RMS normalization
  S   = sum_k x_k^2                       exact, rounded once to float64
  ms  = fl64(S / K)
  r   = fl32(fl64(1 / fl64(sqrt(fl64(ms + eps)))))
  y_k = fl32(fl32(x_k * r) * gamma_k)

Layer normalization (centred)
  mu  = fl64(sum_k x_k / K)               sum exact, rounded once
  d_k = fl64(x_k - mu),  p_k = fl64(d_k * d_k)
  var = fl64(sum_k p_k / K)               sum exact, rounded once
  r   = fl32(fl64(1 / fl64(sqrt(fl64(var + eps)))))
  y_k = fl32(fl32(fl32(x_k - fl32(mu)) * r) * gamma_k + beta_k)   (each op rounded)

then y (binary32) is quantized per 1x128 tile exactly like a bf16 activation:
amax = max |y|, s = fl32(amax / 448), q = E4M3(fl32(y / s)).

Readings where the pages are silent (all stated here): both the centred and the
uncentred (RMS) normalization are offered; the statistics are formed in
float64 from exactly summed terms, so they do not depend on a summation order;
the scaling by r, gamma (and beta) is done in binary32 with the rounding
sequence above; eps is given in binary32 and added in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import math

import numpy as np

from . import bf16, quant


def _exact_row_sums(v64: np.ndarray) -> np.ndarray:
    """Row sums, each exact then rounded once to float64 (math.fsum)."""
    return np.array([math.fsum(row) for row in v64], dtype=np.float64)


def _inv_std(stat: np.ndarray, eps: float) -> np.ndarray:
    e = np.float64(np.float32(eps))
    t = stat + e
    return (np.float64(1.0) / np.sqrt(t)).astype(np.float32)


def rms_norm_f32(x_bits, gamma_bits, eps: float) -> np.ndarray:
    """RMS normalization of bf16 rows -> binary32 (M x K), as in the module docstring."""
    x64 = bf16.to_f64(x_bits)
    M, K = x64.shape
    S = _exact_row_sums(x64 * x64)  # squares of bf16 values are exact in float64
    r = _inv_std(S / np.float64(K), eps)
    x32 = x64.astype(np.float32)
    g32 = bf16.to_f32(gamma_bits)
    return (x32 * r[:, None]) * g32[None, :]


def layer_norm_f32(x_bits, gamma_bits, beta_bits, eps: float) -> np.ndarray:
    """Centred layer normalization of bf16 rows -> binary32 (M x K)."""
    x64 = bf16.to_f64(x_bits)
    M, K = x64.shape
    mu = _exact_row_sums(x64) / np.float64(K)
    d = x64 - mu[:, None]
    var = _exact_row_sums(d * d) / np.float64(K)
    r = _inv_std(var, eps)
    x32 = x64.astype(np.float32)
    xc = x32 - mu.astype(np.float32)[:, None]
    g32 = bf16.to_f32(gamma_bits)
    b32 = bf16.to_f32(beta_bits)
    return ((xc * r[:, None]) * g32[None, :]) + b32[None, :]


def norm_quant_act_1x128(x_bits, gamma_bits, eps: float, beta_bits=None, centred: bool = False):
    """Normalization then the 1x128 quantization of its binary32 output.

    Returns (codes uint8 M x K, scales float32 M x K/128).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.shape[1] % quant.GROUP:
        raise ValueError("K must be a multiple of 128")
    if centred:
        y = layer_norm_f32(x_bits, gamma_bits, beta_bits, eps)
    else:
        y = rms_norm_f32(x_bits, gamma_bits, eps)
    return quant._quant_rows_f32(np.ascontiguousarray(y, dtype=np.float32))
