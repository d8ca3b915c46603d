"""CPU oracle for fine-grained online FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition of what the GPU path computes. Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it. The HIP library never calls it, and it never calls the HIP library: the two
share no code. Inputs reach both sides from the seeded generators, which hold
none of the method's arithmetic.

Sources (the web pages this method is described on; cited by title and passage):

* "Six Reasons Deepseek Ai Is A Waste Of Time" (myomija.com board post):
  - the paragraph on the GEMM operands: FP8 inputs, BF16 or FP32 outputs, and
    E4M3 (4-bit exponent, 3-bit mantissa) on all tensors;
  - the paragraph on standard practice: the maximum absolute value of a tensor
    is mapped to the maximum representable FP8 value;
  - the paragraph on per-group scaling factors along the inner dimension K,
    multiplied in during dequantization on the SIMT cores;
  - the passage on Figure 7 (a): activations grouped per 1x128 tile (per token
    per 128 channels), weights per 128x128 block (per 128 input channels per
    128 output channels);
  - the passage on promotion: MMA partials kept at limited bit width are copied
    to FP32 registers at a fixed interval and accumulated there in full FP32;
  - the preliminary test at K = 4096 in which limited Tensor-Core accumulation
    gives a maximum relative error of nearly 2%.
* codingmall.com knowledge base, Greek page on FP8 in DeepSeek-V3, sections
  "fine-grained quantization", "online quantization" (scales computed from the
  current tile or block, no history of maxima), "increased accumulation
  precision" and "unified E4M3 format".
* codingmall.com knowledge base, Japanese page on FP8 GEMM in DeepSeek-V3,
  items 4-8 (fine-grained quantization, promotion to FP32, unified E4M3, online
  quantization, a GEMM library covering dense and MoE layers).

Modules:
  e4m3     OCP E4M3FN encode/decode at bit level (float64).
  bf16     bfloat16 bits <-> float64 and direct float64 -> bf16 rounding.
  quant    1x128 activation and 128x128 weight quantization.
  gemm     block-scaled GEMM (dense, grouped) as exact per-group float64 sums.
  accsim   limited-precision accumulator model for the K = 4096 demonstration.
  norm     RMS / layer normalization whose binary32 output feeds the 1x128 cast.
  moe      FP8 dispatch: quantize tokens, permute into the padded per-expert layout.
"""

from . import e4m3, bf16, quant, gemm, accsim  # noqa: F401

__all__ = ["e4m3", "bf16", "quant", "gemm", "accsim"]
