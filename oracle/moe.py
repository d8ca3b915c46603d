"""FP8 dispatch of MoE tokens on one GPU: quantize, then permute into the padded
per-expert layout the grouped GEMM consumes.

"Six Reasons Deepseek Ai Is A Waste Of Time", the paragraph on the combine and
dispatch components: activations are quantized to FP8 before the MoE
up-projections and the dispatch then moves FP8 (the combine stays in BF16).
Across GPUs the dispatch is an all-to-all; what one GPU does is this local part:
each token's 1x128 codes and scales are placed in the row block of every expert
the router chose for it. The grouped GEMM's layout (rows of expert e contiguous
from m_offsets[e], every block a multiple of 128 rows, padding rows zero) is
the one of the codingmall.com Japanese page's grouped MoE GEMM (item 8).

What is computed, for x (T tokens x K, bf16) and router choices ids (T x k):
  a slot (t, j) is valid when 0 <= ids[t, j] < G (others are dropped);
  counts[e]   = number of valid slots choosing e
  m_offsets   = 0, then the running sum of counts rounded up to multiples of 128
  the valid slots of expert e, taken in increasing (t, j) order, get rows
  m_offsets[e], m_offsets[e] + 1, ...; row_of_slot[t, j] is that row (-1 when dropped)
  a[row], sa[row] = the 1x128 quantization of x[t] (codes and scales)
  rows m_offsets[e] + counts[e] .. m_offsets[e + 1] - 1 are padding: codes 0, scales 0

Readings where the pages are silent: the order of an expert's rows is the
token order (then the choice index), which makes the layout deterministic;
router choices outside [0, G) are dropped rather than rejected.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

from . import quant

GROUP = 128


def dispatch_1x128(x_bits, topk_ids, G: int):
    """Returns (a codes M_total x K, sa M_total x K/128, m_offsets int32[G+1],
    row_of_slot int32 T x k, counts int64[G])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, K = x_bits.shape
    if ids.shape[0] != T:
        raise ValueError("topk_ids must have one row per token")
    q, s = quant.quant_act_1x128(x_bits)
    valid = (ids >= 0) & (ids < G)
    counts = np.bincount(ids[valid], minlength=G).astype(np.int64)
    padded = (counts + GROUP - 1) // GROUP * GROUP
    offsets = np.zeros(G + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    row_of_slot = np.full(ids.shape, -1, dtype=np.int64)
    next_row = offsets[:-1].copy()
    for t in range(T):
        for j in range(ids.shape[1]):
            if valid[t, j]:
                e = ids[t, j]
                row_of_slot[t, j] = next_row[e]
                next_row[e] += 1
    M_total = int(offsets[-1])
    a = np.zeros((M_total, K), dtype=np.uint8)
    sa = np.zeros((M_total, K // GROUP), dtype=np.float32)
    for t in range(T):
        for j in range(ids.shape[1]):
            r = row_of_slot[t, j]
            if r >= 0:
                a[r] = q[t]
                sa[r] = s[t]
    return a, sa, offsets.astype(np.int32), row_of_slot.astype(np.int32), counts


def max_rows(T: int, k: int, G: int) -> int:
    """Upper bound on m_offsets[G] (every expert adds at most 127 padding rows),
    rounded up to a multiple of 128."""
    return (T * k + (GROUP - 1) * G + GROUP - 1) // GROUP * GROUP
