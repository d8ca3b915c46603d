"""fp8_fine_grained_online_amd: fine-grained online FP8 quantization and the
block-scaled FP8 GEMM on AMD MI355X (gfx950).

The compute path is the HIP library ``libfp8q.so`` (C ABI, ``include/fp8q.h``).
This module only marshals arguments: it checks tensor dtypes/devices/layouts,
allocates outputs with torch when the caller does not pass them, and forwards
raw device pointers and torch's current HIP stream. There is no other path:
if the library is missing, every call raises.

Entry points (same names as the C ABI):
  fp8q_quant_act_1x128(x)                    -> (q, sa)
  fp8q_quant_act_1x128_nt(x)                 -> (q, sa)   same, non-temporal stores
  fp8q_quant_weight_128x128(w)               -> (q, sb)
  fp8_gemm_blockscaled(a, sa, b, sb, out_dtype)          -> c
  fp8_gemm_blockscaled_ws(a, sa, b, sb, out_dtype)       -> c   (split-K for small M)
  fp8_gemm_blockscaled_noalloc(a, sa, b, sb, out_dtype)  -> c   (same, library scratch: no allocation)
  fp8_gemm_blockscaled_bf16a(a_bf16, b, sb, out_dtype)   -> c [, qa, sa]   quantize-on-load
  fp8_gemm_grouped(a, sa, b, sb, m_offsets, out_dtype)   -> c
  fp8q_norm_quant_act_1x128(x, gamma, eps, beta, centred) -> (q, sa)   normalization + cast
  fp8q_moe_dispatch_1x128(x, topk_ids, G) -> (q, sa, m_offsets, row_of_slot)   MoE FP8 dispatch
Backward pass (Dgrad dX = dY W, Wgrad dW = dY^T X):
  fp8q_quant_act_128x1(x)                    -> (qt, st)   128x1 tiles, transposed
  fp8q_quant_act_1x128_128x1(x)              -> (q, sa, qt, st)   both, one read of x
  fp8q_requant_1x128_to_128x1(q, sa)         -> (qt, st)
  fp8q_transpose_weight_128x128(q, sb)       -> (qt, sbt)
  fp8_gemm_rowscaled(a, sa, b, sb, out_dtype)            -> c
"""

from ._lib import (  # noqa: F401
    Fp8qError,
    FP8Q_OUT_BF16,
    FP8Q_OUT_F32,
    STATUS,
    fp8_gemm_blockscaled,
    fp8_gemm_blockscaled_bf16a,
    fp8_gemm_blockscaled_noalloc,
    fp8_gemm_blockscaled_ws,
    fp8_gemm_grouped,
    fp8_gemm_rowscaled,
    fp8q_quant_act_128x1,
    fp8q_quant_act_1x128_128x1,
    fp8q_norm_quant_act_1x128,
    fp8q_moe_dispatch_1x128,
    fp8q_quant_act_1x128,
    fp8q_quant_act_1x128_nt,
    fp8q_requant_1x128_to_128x1,
    fp8q_transpose_weight_128x128,
    fp8q_quant_weight_128x128,
    fp8q_version,
    lib,
    lib_path,
)

__all__ = [
    "Fp8qError", "FP8Q_OUT_BF16", "FP8Q_OUT_F32", "STATUS",
    "fp8q_quant_act_1x128", "fp8q_quant_act_1x128_nt", "fp8q_quant_weight_128x128",
    "fp8_gemm_blockscaled", "fp8_gemm_blockscaled_bf16a", "fp8_gemm_blockscaled_ws", "fp8_gemm_blockscaled_noalloc", "fp8_gemm_grouped", "fp8q_version", "lib", "lib_path",
    "fp8q_quant_act_128x1", "fp8q_quant_act_1x128_128x1", "fp8q_norm_quant_act_1x128", "fp8q_moe_dispatch_1x128", "fp8q_requant_1x128_to_128x1", "fp8q_transpose_weight_128x128",
    "fp8_gemm_rowscaled",
]
