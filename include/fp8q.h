/*
 * fp8q: fine-grained online FP8 quantization and block-scaled FP8 GEMM for
 * AMD MI355X (gfx950). C ABI.
 *
 * Method (as described on the source pages):
 *  - "Six Reasons Deepseek Ai Is A Waste Of Time" (myomija.com):
 *      * GEMMs take FP8 (E4M3) operands and produce BF16 or FP32 outputs
 *        (paragraph on the GEMM operands);
 *      * activations are scaled per 1x128 tile (per token per 128 channels),
 *        weights per 128x128 block (per 128 input x 128 output channels)
 *        (passage on Figure 7 (a));
 *      * the scale maps the maximum absolute value to the largest FP8 value
 *        (paragraph on standard practice);
 *      * per-group scaling factors along K are applied while dequantizing MMA
 *        partials, which are promoted to FP32 accumulators at a fixed interval
 *        (paragraphs on fine-grained quantization and on promotion).
 *  - codingmall.com, Greek page on FP8 in DeepSeek-V3, section "online
 *    quantization": scales are computed on the fly from the current tile/block.
 *  - codingmall.com, Japanese page on FP8 GEMM in DeepSeek-V3, item 8: dense
 *    and MoE (grouped) GEMMs.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *    unless stated otherwise. The caller owns and allocates every buffer; the
 *    library allocates nothing and keeps no mutable global state.
 *  - All matrices are row-major with the K (reduction) dimension contiguous.
 *    Activations A are M x K, weights B are N x K (out-channels x in-channels);
 *    the GEMM computes C = A * B^T, C is M x N.
 *  - Codes are OCP E4M3FN bytes (max finite 448, 0x7F/0xFF NaN).
 *  - Scales are float32 dequantization factors s = fl32(amax / 448): a code
 *    times its scale approximates the original value. An all-zero tile or
 *    block has scale 0 and zero codes (the sign of each zero is kept).
 *  - Each call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns once the kernels are enqueued. Calls are reentrant.
 *  - Errors: a nonzero fp8q_status. Argument checks run on the host before any
 *    HIP call; a failing check launches nothing. Launch failures return
 *    FP8Q_ERR_LAUNCH. A fault inside a kernel surfaces as an error at the
 *    caller's next synchronization. Nothing aborts, throws or prints.
 *  - Non-finite inputs are outside the contract (codes and outputs are then
 *    unspecified, but every kernel still terminates).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#if defined(__GNUC__)
#define FP8Q_API __attribute__((visibility("default")))
#else
#define FP8Q_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8Q_OK = 0,
  FP8Q_ERR_NULL = 1,      /* a required pointer is NULL */
  FP8Q_ERR_SHAPE = 2,     /* negative size, or K/N not a multiple of 128, or G < 1 */
  FP8Q_ERR_ALIGN = 3,     /* code/input/output pointers need 16-byte, scales 4-byte alignment */
  FP8Q_ERR_DTYPE = 4,     /* out_dtype not one of fp8q_out_dtype */
  FP8Q_ERR_LAUNCH = 5,    /* the HIP runtime refused a launch */
  FP8Q_ERR_NO_DEVICE = 6, /* no usable gfx950 device */
  FP8Q_ERR_TOO_LARGE = 7  /* a size overflows the kernels' 32-bit tile indexing */
} fp8q_status;

typedef enum { FP8Q_OUT_F32 = 0, FP8Q_OUT_BF16 = 1 } fp8q_out_dtype;

/* Library version: major * 10000 + minor * 100 + patch. */
FP8Q_API int fp8q_version(void);

/* Static text for a status code (never NULL). */
FP8Q_API const char* fp8q_status_string(int status);

/*
 * Online 1x128 activation quantization.
 * Source: the Figure 7 (a) passage ("per token per 128 channels") and the
 * standard-practice paragraph of "Six Reasons Deepseek Ai Is A Waste Of Time";
 * "online quantization" on the Greek codingmall.com page.
 *
 * For each row m and K-group g (128 consecutive columns):
 *   amax = max |x[m, 128g .. 128g+127]|, s = fl32(amax / 448),
 *   q[m, k] = E4M3_RNE(clamp(fl32(x[m, k] / s), -448, 448)),  sa[m, g] = s.
 *
 *   x_bf16 : in,  M x K bfloat16, 16-byte aligned
 *   q      : out, M x K E4M3 bytes, 16-byte aligned
 *   sa     : out, M x (K/128) float32, 4-byte aligned
 * Requires K % 128 == 0. M == 0 or K == 0 is a no-op returning FP8Q_OK.
 */
FP8Q_API int fp8q_quant_act_1x128(const void* x_bf16, int64_t M, int64_t K, uint8_t* q, float* sa,
                         void* stream);

/*
 * 128x128 weight quantization: as above with amax over each 128x128 block.
 * Source: the Figure 7 (a) passage ("per 128 input channels per 128 output
 * channels") of "Six Reasons Deepseek Ai Is A Waste Of Time".
 *
 *   w_bf16 : in,  N x K bfloat16 (for G experts pass N = G * N_e: the blocks
 *            never straddle experts when N_e % 128 == 0)
 *   q      : out, N x K E4M3 bytes
 *   sb     : out, (N/128) x (K/128) float32
 * Requires N % 128 == 0 and K % 128 == 0. N == 0 or K == 0 is a no-op.
 */
FP8Q_API int fp8q_quant_weight_128x128(const void* w_bf16, int64_t N, int64_t K, uint8_t* q, float* sb,
                              void* stream);

/*
 * Block-scaled FP8 GEMM: C = A * B^T with per-group promotion.
 * Source: the paragraphs on the GEMM operands, on fine-grained quantization
 * and on promotion in "Six Reasons Deepseek Ai Is A Waste Of Time".
 *
 *   P_g[m, n] = sum_{k in group g} dec(a[m, k]) * dec(b[n, k])  (FP8 MFMA, FP32)
 *   acc[m, n] += (sa[m, g] * sb[n / 128, g]) * P_g[m, n]         (FP32 VALU)
 *   c[m, n] = acc (float32) or RNE_bf16(acc)
 *
 *   a  : in,  M x K E4M3 (from fp8q_quant_act_1x128), 16-byte aligned
 *   sa : in,  M x (K/128) float32
 *   b  : in,  N x K E4M3 (from fp8q_quant_weight_128x128), 16-byte aligned
 *   sb : in,  (N/128) x (K/128) float32
 *   c  : out, M x N, float32 or bfloat16 per out_dtype, 16-byte aligned
 * Requires N % 128 == 0, K % 128 == 0; M is arbitrary (a ragged last tile is
 * masked). M == 0 or N == 0 is a no-op; K == 0 writes zeros (and reads no
 * operand, so a, sa, b, sb may then be NULL).
 */
FP8Q_API int fp8_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                         void* c, int out_dtype, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Grouped (MoE) block-scaled FP8 GEMM: expert e owns rows
 * [m_offsets[e], m_offsets[e+1]) of A and C and multiplies them by its own
 * weights B_e with scales sb_e, exactly as fp8_gemm_blockscaled would.
 * Source: item 8 of the Japanese codingmall.com page (dense and MoE GEMMs),
 * with the per-expert arithmetic of fp8_gemm_blockscaled.
 *
 *   a         : in,  M_total x K E4M3, experts' rows contiguous
 *   sa        : in,  M_total x (K/128) float32
 *   b         : in,  G x N x K E4M3
 *   sb        : in,  G x (N/128) x (K/128) float32
 *   c         : out, M_total x N (float32 or bfloat16)
 *   m_offsets : in,  DEVICE int32[G+1]; m_offsets[0] = 0, nondecreasing,
 *               every entry a multiple of 128, m_offsets[G] = M_total
 *   M_total   : host copy of m_offsets[G] (sizes the launch; no device read)
 * Offsets that break these rules are outside the contract: rows are then
 * assigned to experts by the (clamped) offsets, and no access leaves the
 * buffers sized by M_total, G, N and K.
 */
FP8Q_API int fp8_gemm_grouped(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                     void* c, int out_dtype, const int32_t* m_offsets, int64_t G,
                     int64_t M_total, int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
