"""Online fine-grained FP8 quantization: 1x128 activation tiles, 128x128 weight blocks.

What is computed (for every tile of an activation, every block of a weight):

  amax = max |x| over the tile/block                 (exact)
  s    = fl32(amax / 448)                            (IEEE binary32 division)
  q    = E4M3(fl32(x / s)) for each x in the tile    (RNE, saturating at 448)
  an all-zero tile has s = 0 and codes +0 / -0 (the sign of x).

Sources:
* "Six Reasons Deepseek Ai Is A Waste Of Time" (myomija.com), the passage on
  Figure 7 (a): activations are grouped and scaled per 1x128 tile (per token per
  128 channels) and weights per 128x128 block (per 128 input channels per 128
  output channels); the paragraph on standard practice: the maximum absolute
  value is scaled to the largest representable FP8 value (448 for E4M3FN).
* codingmall.com, Greek page on FP8 in DeepSeek-V3, section "online
  quantization" (and item 7 of the Japanese page): the scale of each tile or
  block is computed on the fly from its current values, with no delayed
  (history-of-maxima) scaling.

Readings where the pages are silent: the stored scale is the dequantization
factor amax/448 (a code times s gives back x); the per-element quotient is the
correctly rounded binary32 x/s; an all-zero tile gets scale 0.

Inputs are raw bf16 bit patterns (uint16 arrays) so that every consumer sees the
same bytes; layouts are row-major with K contiguous.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

from . import bf16, e4m3

GROUP = 128
FP8_MAX = np.float32(448.0)


def _quantize_groups(x32: np.ndarray, amax: np.ndarray):
    """x32: float32 values; amax: float32 maxima broadcastable to x32."""
    s = (amax / FP8_MAX).astype(np.float32)  # one IEEE binary32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (x32 / s).astype(np.float32)  # IEEE binary32 division per element
    q = np.where(s == 0, x32, q)  # zero tile: x is +-0, keep its sign
    codes = e4m3.encode(q.astype(np.float64))
    return codes, s


def quant_act_1x128(x_bits: np.ndarray):
    """Activations M x K (bf16 bits) -> (codes uint8 M x K, scales float32 M x K/128)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    x = bf16.to_f32(x_bits).reshape(M, K // GROUP, GROUP)
    amax = np.max(np.abs(x), axis=2, keepdims=True)
    codes, s = _quantize_groups(x, amax)
    return codes.reshape(M, K), s.reshape(M, K // GROUP)


def quant_weight_128x128(w_bits: np.ndarray):
    """Weights N x K (bf16 bits) -> (codes uint8 N x K, scales float32 N/128 x K/128)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if K % GROUP or N % GROUP:
        raise ValueError("N and K must be multiples of 128")
    w = bf16.to_f32(w_bits).reshape(N // GROUP, GROUP, K // GROUP, GROUP)
    amax = np.max(np.abs(w), axis=(1, 3), keepdims=True)
    codes, s = _quantize_groups(w, amax)
    return codes.reshape(N, K), s.reshape(N // GROUP, K // GROUP)


def quant_act_128x1(x_bits: np.ndarray):
    """Activations M x K (bf16 bits) in 128x1 tiles (128 consecutive rows of one
    column), returned transposed: (codes uint8 K x M, scales float32 K x M/128).

    The backward pass regroups activations from 1x128 to 128x1 tiles ("Six
    Reasons Deepseek Ai Is A Waste Of Time", the sentence next to the Figure 7 (a)
    passage); a 128x1 tile of X is a 1x128 tile of X^T, and the transposed layout
    is the one a GEMM reducing over M consumes.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if M % GROUP:
        raise ValueError("M must be a multiple of 128")
    return quant_act_1x128(np.ascontiguousarray(x_bits.T))


def _quant_rows_f32(x32: np.ndarray):
    """1x128 quantization of float32 rows (same rule as for bf16 inputs)."""
    R, C = x32.shape
    x = x32.reshape(R, C // GROUP, GROUP)
    amax = np.max(np.abs(x), axis=2, keepdims=True)
    codes, s = _quantize_groups(x, amax)
    return codes.reshape(R, C), s.reshape(R, C // GROUP)


def requant_1x128_to_128x1(codes: np.ndarray, scales: np.ndarray):
    """Stored 1x128 FP8 activations -> 128x1 tiles, transposed (K x M codes).

    The pages store the forward activations as 1x128 FP8 tiles (woojincopolymer.co.kr
    post, memory paragraph; "Six Reasons Deepseek Ai Is A Waste Of Time" on
    compressing cached activations) and convert them to 128x1 tiles for the
    backward pass (the sentence next to the Figure 7 (a) passage of the latter).
    Reading: each element is dequantized to binary32, v = fl32(dec(q) * s)
    (one rounding of the exact product), and v^T is quantized in 1x128 tiles
    with the usual rule.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    M, K = codes.shape
    if M % GROUP or K % GROUP:
        raise ValueError("M and K must be multiples of 128")
    v = (e4m3.decode(codes).reshape(M, K // GROUP, GROUP)
         * np.asarray(scales, np.float64)[:, :, None]).astype(np.float32).reshape(M, K)
    return _quant_rows_f32(np.ascontiguousarray(v.T))


def transpose_weight_128x128(codes: np.ndarray, scales: np.ndarray):
    """W (N x K codes, N/128 x K/128 scales) -> W^T (K x N codes, K/128 x N/128).

    A 128x128 block of W is a 128x128 block of W^T with the same scale, so the
    transpose is exact; it is the weight operand of the input-gradient GEMM.
    """
    return (np.ascontiguousarray(np.asarray(codes).T),
            np.ascontiguousarray(np.asarray(scales, np.float32).T))


def dequant_act(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes * s per 1x128 tile, exact in float64."""
    M, K = codes.shape
    v = e4m3.decode(codes).reshape(M, K // GROUP, GROUP)
    return (v * scales.astype(np.float64)[:, :, None]).reshape(M, K)


def dequant_weight(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes * s per 128x128 block, exact in float64."""
    N, K = codes.shape
    v = e4m3.decode(codes).reshape(N // GROUP, GROUP, K // GROUP, GROUP)
    return (v * scales.astype(np.float64)[:, None, :, None]).reshape(N, K)
