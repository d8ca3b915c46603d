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
 *  - Size limits (FP8Q_ERR_TOO_LARGE beyond them): every dimension below 2^31;
 *    the GEMMs' reduction dimension K at most 2^23 (operand tiles are
 *    addressed with 32-bit offsets).
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
  FP8Q_ERR_TOO_LARGE = 7, /* a size overflows the kernels' 32-bit tile indexing */
  FP8Q_ERR_SCRATCH = 8    /* fp8_gemm_blockscaled_noalloc: the partials exceed its static scratch */
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
 * q and sa are written with ordinary stores, so a GEMM that reads them next
 * finds them in the GPU's 256 MB Infinity Cache; codes larger than that cache
 * (M * K > 256 MiB) cannot stay there and go out with non-temporal stores.
 */
FP8Q_API int fp8q_quant_act_1x128(const void* x_bf16, int64_t M, int64_t K, uint8_t* q, float* sa,
                         void* stream);

/*
 * fp8q_quant_act_1x128 with non-temporal stores: the same codes and scales,
 * bit for bit, with the same arguments, requirements and errors. The stores
 * do not keep q and sa in the GPU's 256 MB Infinity Cache, which raises the
 * kernel's HBM throughput (16384 x 7168 on MI355X: 6.4 TB/s against 5.9).
 * Use it for activations that are not read next on this GPU (codes sent to
 * another GPU, or written out); above 256 MiB of codes fp8q_quant_act_1x128
 * stores this way by itself. For codes that a GEMM reads next, the cached
 * form is faster overall, because the GEMM then finds its operand in the
 * cache. (4096^3: quantization plus GEMM is about 11 us slower with
 * non-temporal codes.) Same source passages as fp8q_quant_act_1x128.
 */
FP8Q_API int fp8q_quant_act_1x128_nt(const void* x_bf16, int64_t M, int64_t K, uint8_t* q,
                                     float* sa, void* stream);

/*
 * 128x128 weight quantization: as above with amax over each 128x128 block.
 * Source: the Figure 7 (a) passage of "Six Reasons Deepseek Ai Is A Waste Of
 * Time" (weights grouped in blocks of 128 input by 128 output channels).
 *
 *   w_bf16 : in,  N x K bfloat16 (for G experts pass N = G * N_e: the blocks
 *            never straddle experts when N_e % 128 == 0)
 *   q      : out, N x K E4M3 bytes
 *   sb     : out, (N/128) x (K/128) float32
 * Requires N % 128 == 0 and K % 128 == 0. N == 0 or K == 0 is a no-op.
 * Store policy as for fp8q_quant_act_1x128: non-temporal when N * K > 256 MiB.
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
 * fp8_gemm_blockscaled with a caller workspace, for small-M shapes (few rows,
 * e.g. 64 x 7168 x 7168). There the plain call's kernel gives every
 * workgroup 32 columns, so every workgroup re-reads all of A; with a
 * workspace the K groups are split across workgroups of 64 x 128 (A is read
 * 4x less often) and the FP32 partials of the splits are summed, in split
 * order, by a second kernel before the output rounding. Same arithmetic and
 * the same results up to the FP32 summation order (within the tolerance of
 * fp8_gemm_blockscaled); deterministic.
 * Source: as fp8_gemm_blockscaled.
 *
 *   workspace, workspace_bytes : DEVICE scratch of at least
 *     fp8_gemm_blockscaled_ws_bytes(M, N, K) bytes, 16-byte aligned, owned by
 *     the caller, no contents needed on entry. When that size is 0 the shape
 *     does not take the split path and the call is fp8_gemm_blockscaled
 *     (workspace may then be NULL): shapes with fewer than 16 K groups
 *     (K < 2048), or too many tiles for two splits. The size is 4 * S * M * N
 *     for S splits (S <= 256 / number of 64 x 128 tiles). Two calls in flight
 *     at once on one workspace (different streams) race.
 */
FP8Q_API int fp8_gemm_blockscaled_ws(const uint8_t* a, const float* sa, const uint8_t* b,
                                     const float* sb, void* c, int out_dtype, int64_t M, int64_t N,
                                     int64_t K, void* workspace, int64_t workspace_bytes,
                                     void* stream);

/*
 * Quantize-on-load GEMM: C = Q(A) * B^T with A given in bf16, where Q is the
 * 1x128 activation quantization of fp8q_quant_act_1x128, done inside the
 * GEMM's load stage (each K group of A is read in bf16, quantized in
 * registers and written to LDS as E4M3 codes + scale for the matrix cores).
 * Results equal fp8q_quant_act_1x128 followed by fp8_gemm_blockscaled: the
 * same codes and scales, the same per-group promotion (up to the FP32
 * summation order of the MFMAs, within that call's tolerance).
 * Source: the woojincopolymer.co.kr post, paragraph of hardware suggestions
 * (fuse the FP8 cast with the global-to-shared transfer); the arithmetic of
 * fp8q_quant_act_1x128 and fp8_gemm_blockscaled.
 *
 *   a_bf16 : in,  M x K bf16, row-major, 16-byte aligned
 *   b, sb  : in,  as for fp8_gemm_blockscaled (N x K E4M3, (N/128) x (K/128))
 *   c      : out, M x N (float32 or bfloat16 per out_dtype), 16-byte aligned
 *   qa, sa : optional outputs (both NULL or both set): the codes (M x K,
 *            16-byte aligned) and scales (M x (K/128)) of A, bit-identical to
 *            fp8q_quant_act_1x128's; written when M, N and K are all > 0
 * Requires N % 128 == 0 and K % 128 == 0; M arbitrary. M == 0 or N == 0 is a
 * no-op; K == 0 writes zeros to c. Each of the N/256 column tiles quantizes
 * its rows of A again (the price of the fusion on this hardware).
 */
FP8Q_API int fp8_gemm_blockscaled_bf16a(const void* a_bf16, const uint8_t* b, const float* sb,
                                        void* c, int out_dtype, int64_t M, int64_t N, int64_t K,
                                        uint8_t* qa, float* sa, void* stream);

/* Workspace bytes fp8_gemm_blockscaled_ws needs for this shape (0: none; -1: invalid). */
FP8Q_API int64_t fp8_gemm_blockscaled_ws_bytes(int64_t M, int64_t N, int64_t K);

/*
 * fp8_gemm_blockscaled_ws without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The split-K partials go to an 8 MiB
 * array the library keeps in device memory, one per GPU it runs on, held
 * until the process ends. Same kernels, same results bit for bit as
 * fp8_gemm_blockscaled_ws; arguments as for fp8_gemm_blockscaled.
 *
 * The partials of S splits of 64 x 128 tiles take 4 * S * M * N bytes with at
 * most 256 split tiles, so never more than 256 * 64 * 128 * 4 = 8 MiB
 * (64 x 7168 x 7168: 7.0 MiB); FP8Q_ERR_SCRATCH (a call needing more than
 * 8388608 bytes) guards that bound. Shapes whose workspace size is 0 run
 * fp8_gemm_blockscaled. The call allocates nothing (no hipMalloc, no
 * allocating library routine); it looks up the current device's copy of the
 * array once per device. All calls on one GPU share that GPU's copy: two
 * calls in flight at once on one GPU (different streams) race on it. Its
 * contents need not start at any value (every partial is written before it
 * is read).
 */
FP8Q_API int fp8_gemm_blockscaled_noalloc(const uint8_t* a, const float* sa, const uint8_t* b,
                                          const float* sb, void* c, int out_dtype, int64_t M,
                                          int64_t N, int64_t K, void* stream);

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
 *               every entry a multiple of 128, m_offsets[G] <= M_total
 *   M_total   : host-side row count of a and c, at least m_offsets[G] (sizes
 *               the launch; no device read). Rows from m_offsets[G] to
 *               M_total are neither read nor written, so the output of
 *               fp8q_moe_dispatch_1x128 can be passed with its capacity as
 *               M_total and no host synchronization.
 * Offsets that break these rules are outside the contract: rows are then
 * assigned to experts by the (clamped) offsets, and no access leaves the
 * buffers sized by M_total, G, N and K.
 */
FP8Q_API int fp8_gemm_grouped(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                     void* c, int out_dtype, const int32_t* m_offsets, int64_t G,
                     int64_t M_total, int64_t N, int64_t K, void* stream);

/*
 * FP8 dispatch of MoE tokens on one GPU: quantize every token once (1x128
 * tiles, the rule of fp8q_quant_act_1x128) and place its codes and scales in
 * the row block of each expert the router chose, in the padded per-expert
 * layout fp8_gemm_grouped consumes.
 * Source: "Six Reasons Deepseek Ai Is A Waste Of Time", the paragraph on the
 * combine and dispatch components (activations quantized to FP8 before the
 * MoE up-projections, then dispatched); the grouped layout of item 8 of the
 * Japanese codingmall.com page. The all-to-all between GPUs is not part of
 * this call.
 *
 * A slot (t, j) = topk_ids[t * topk + j] is valid when 0 <= id < G; invalid
 * choices are dropped. counts[e] = valid slots choosing e;
 * m_offsets[0] = 0, m_offsets[e+1] = m_offsets[e] + roundup(counts[e], 128).
 * Expert e's valid slots, in increasing slot order, take rows m_offsets[e],
 * m_offsets[e] + 1, ...; row_of_slot[t * topk + j] is that row, or -1.
 * Row r of (q, sa) holds the 1x128 codes and scales of its token; the padding
 * rows m_offsets[e] + counts[e] .. m_offsets[e+1]-1 are zero (codes and
 * scales). Rows from m_offsets[G] to M_cap are not written.
 *
 *   x_bf16      : in,  T x K bfloat16, 16-byte aligned
 *   topk_ids    : in,  DEVICE int32 T x topk, 4-byte aligned
 *   q, sa       : out, M_cap x K E4M3 (16-byte aligned), M_cap x (K/128) float32
 *   M_cap       : rows of q and sa; at least fp8q_moe_dispatch_max_rows(T, topk, G)
 *                 = T * topk + 127 * G (the largest possible m_offsets[G])
 *                 rounded up to a multiple of 128
 *   m_offsets   : out, DEVICE int32[G+1]
 *   row_of_slot : out, DEVICE int32 T x topk (the map a combine step inverts)
 *   workspace   : DEVICE scratch of at least
 *                 fp8q_moe_dispatch_workspace_bytes(T, topk, G) bytes, 4-byte
 *                 aligned, owned by the caller; no contents needed on entry
 * Requires K % 128 == 0, topk >= 1, 1 <= G <= 1024. T == 0 still writes
 * m_offsets (all zero). Up to three kernels are enqueued on `stream`: count
 * (per-block histograms, and each slot's rank inside its block, held in
 * row_of_slot until the last kernel), scan and quantize/scatter, which also
 * turns the ranks into rows (only the scan when T == 0; with K == 0 the last
 * kernel only writes the row map).
 */
FP8Q_API int fp8q_moe_dispatch_1x128(const void* x_bf16, const int32_t* topk_ids, int64_t T,
                                     int64_t K, int64_t topk, int64_t G, uint8_t* q, float* sa,
                                     int64_t M_cap, int32_t* m_offsets, int32_t* row_of_slot,
                                     void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of device workspace fp8q_moe_dispatch_1x128 needs (-1 for invalid sizes). */
FP8Q_API int64_t fp8q_moe_dispatch_workspace_bytes(int64_t T, int64_t topk, int64_t G);

/* Rows the dispatch outputs must hold: T * topk + 127 * G rounded up to a
 * multiple of 128, a valid M_total for fp8_gemm_grouped (-1 for invalid sizes). */
FP8Q_API int64_t fp8q_moe_dispatch_max_rows(int64_t T, int64_t topk, int64_t G);

/*
 * Layer normalization fused with the 1x128 activation quantization.
 * Source: the woojincopolymer.co.kr post, paragraph of hardware suggestions
 * (a warp-level cast to fuse layer normalization with the FP8 cast), and
 * "Six Reasons Deepseek Ai Is A Waste Of Time" (normalization kept in higher
 * precision while the GEMMs run in FP8).
 *
 * Per row x (K values), with statistics from exact sums rounded once to
 * float64 and every float64 step correctly rounded:
 *   centred = 0 (RMS):   r = fl32(1 / sqrt(fl64(sum x^2 / K) + eps)),
 *                        y = fl32(fl32(x * r) * gamma)
 *   centred = 1 (layer): mu = fl64(sum x / K),
 *                        var = fl64(sum fl64(fl64(x - mu)^2) / K),
 *                        r = fl32(1 / sqrt(var + eps)),
 *                        y = fl32(fl32(fl32(fl32(x - fl32(mu)) * r) * gamma) + beta)
 * then y (binary32, never stored) is quantized per 1x128 tile exactly like
 * fp8q_quant_act_1x128 quantizes its input.
 *
 *   x_bf16     : in,  M x K bfloat16, 16-byte aligned
 *   gamma_bf16 : in,  K bfloat16 scale, 16-byte aligned
 *   beta_bf16  : in,  K bfloat16 shift (centred = 1 only; may be NULL otherwise)
 *   eps        : finite, >= 0 (a zero row with eps = 0 gives non-finite values,
 *                outside the contract)
 *   q, sa      : out, M x K E4M3 (16-byte aligned), M x (K/128) float32
 * Requires K % 128 == 0 and K <= 16384 (a row lives in one wavefront's
 * registers). M == 0 or K == 0 is a no-op.
 */
FP8Q_API int fp8q_norm_quant_act_1x128(const void* x_bf16, const void* gamma_bf16,
                                       const void* beta_bf16, float eps, int centred, int64_t M,
                                       int64_t K, uint8_t* q, float* sa, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Backward pass of a linear layer Y = X W^T (X: M tokens x K in-channels,
 * W: N out-channels x K). "Six Reasons Deepseek Ai Is A Waste Of Time": the
 * GEMM-operands paragraph (Fprop, Dgrad and Wgrad all in E4M3) and the
 * Figure 7 (a) passage (activations converted from 1x128 to 128x1 tiles for
 * the backward pass); woojincopolymer.co.kr post, memory paragraph (the
 * forward activations are stored as 1x128 FP8 tiles).
 *
 *   Dgrad  dX = dY W    : fp8q_quant_act_1x128(dY) and
 *                         fp8q_transpose_weight_128x128(W) feed
 *                         fp8_gemm_blockscaled (A = dY, B = W^T, K = N).
 *   Wgrad  dW = dY^T X  : fp8q_quant_act_128x1(dY) and
 *                         fp8q_requant_1x128_to_128x1(stored X) feed
 *                         fp8_gemm_rowscaled (A = dY^T, B = X^T, K = M).
 *   fp8q_quant_act_1x128_128x1(dY) produces both quantizations of dY at once.
 * ---------------------------------------------------------------------------
 */

/*
 * 128x1 activation quantization, output transposed.
 * Source: the Figure 7 (a) passage of "Six Reasons Deepseek Ai Is A Waste Of
 * Time" (128x1 tiles in the backward pass), with the quantization rule of
 * fp8q_quant_act_1x128.
 *
 * A 128x1 tile is 128 consecutive rows of one column of x. For each column k
 * and row group r (rows 128r .. 128r+127):
 *   amax = max |x[128r .. 128r+127, k]|, s = fl32(amax / 448),
 *   qt[k, m] = E4M3_RNE(clamp(fl32(x[m, k] / s), -448, 448)),  st[k, r] = s.
 * i.e. the 1x128 quantization of x^T.
 *
 *   x_bf16 : in,  M x K bfloat16, 16-byte aligned
 *   qt     : out, K x M E4M3 bytes (x^T), 16-byte aligned
 *   st     : out, K x (M/128) float32, 4-byte aligned
 * Requires M % 128 == 0 and K % 128 == 0. M == 0 or K == 0 is a no-op.
 */
FP8Q_API int fp8q_quant_act_128x1(const void* x_bf16, int64_t M, int64_t K, uint8_t* qt, float* st,
                                  void* stream);

/*
 * Both quantizations of one activation (or output-gradient) tensor from a
 * single read of it: the 1x128 result of fp8q_quant_act_1x128 (q, sa) and
 * the transposed 128x1 result of fp8q_quant_act_128x1 (qt, st), bit for bit.
 * Dgrad consumes dY in 1x128 tiles and Wgrad in 128x1 tiles (sources as for
 * those two calls), so dY is read from memory once instead of twice.
 *
 *   x_bf16 : in,  M x K bfloat16, 16-byte aligned
 *   q, sa  : out, M x K E4M3 (16-byte aligned) and M x (K/128) float32
 *   qt, st : out, K x M E4M3 (16-byte aligned) and K x (M/128) float32
 * Requires M % 128 == 0 and K % 128 == 0. M == 0 or K == 0 is a no-op.
 */
FP8Q_API int fp8q_quant_act_1x128_128x1(const void* x_bf16, int64_t M, int64_t K, uint8_t* q,
                                        float* sa, uint8_t* qt, float* st, void* stream);

/*
 * Re-tiling of stored 1x128 FP8 activations into 128x1 tiles, transposed.
 * Source: the Figure 7 (a) passage of "Six Reasons Deepseek Ai Is A Waste Of
 * Time" (conversion from 1x128 to 128x1 tiles) and the memory paragraph of
 * the woojincopolymer.co.kr post (the stored form is 1x128 FP8).
 *
 * Each element is dequantized to binary32 with one rounding,
 *   v[m, k] = fl32(dec(q[m, k]) * sa[m, k/128]),
 * and v is quantized in 128x1 tiles exactly as fp8q_quant_act_128x1 does
 * (amax over 128 rows of a column, s = fl32(amax/448), codes of fl32(v/s)).
 *
 *   q  : in,  M x K E4M3 (from fp8q_quant_act_1x128), 16-byte aligned
 *   sa : in,  M x (K/128) float32; every dec(q) * sa must be finite in
 *        binary32 (true for any output of fp8q_quant_act_1x128 on finite
 *        input: |dec(q)| <= 448 and sa <= FLT_MAX / 448)
 *   qt : out, K x M E4M3, 16-byte aligned
 *   st : out, K x (M/128) float32
 * Requires M % 128 == 0 and K % 128 == 0. M == 0 or K == 0 is a no-op.
 */
FP8Q_API int fp8q_requant_1x128_to_128x1(const uint8_t* q, const float* sa, int64_t M, int64_t K,
                                         uint8_t* qt, float* st, void* stream);

/*
 * Transpose of 128x128-block-quantized weights: W (N x K) -> W^T (K x N).
 * A 128x128 block of W is a 128x128 block of W^T with the same maximum, so
 * the transposed codes and scales are exactly those of quantizing W^T; the
 * result is the weight operand of the Dgrad GEMM. Source: the Figure 7 (a)
 * passage of "Six Reasons Deepseek Ai Is A Waste Of Time" (128x128 blocks)
 * and its GEMM-operands paragraph (Dgrad in E4M3).
 *
 *   q   : in,  N x K E4M3, 16-byte aligned
 *   sb  : in,  (N/128) x (K/128) float32
 *   qt  : out, K x N E4M3, 16-byte aligned
 *   sbt : out, (K/128) x (N/128) float32
 * Requires N % 128 == 0 and K % 128 == 0. N == 0 or K == 0 is a no-op.
 */
FP8Q_API int fp8q_transpose_weight_128x128(const uint8_t* q, const float* sb, int64_t N, int64_t K,
                                           uint8_t* qt, float* sbt, void* stream);

/*
 * FP8 GEMM with 1x128 scales on both operands (the Wgrad GEMM): C = A * B^T,
 *   acc[m, n] += (sa[m, g] * sb[n, g]) * P_g[m, n],
 * with P_g and the promotion as in fp8_gemm_blockscaled. Source: the
 * GEMM-operands paragraph (Wgrad in E4M3) and the paragraphs on fine-grained
 * quantization and promotion of "Six Reasons Deepseek Ai Is A Waste Of Time";
 * both operands are activations/gradients quantized along the reduction
 * dimension (the 128x1 tiles of the Figure 7 (a) passage, stored transposed).
 *
 *   a  : in,  M x K E4M3, 16-byte aligned   (Wgrad: dY^T, M = out-channels)
 *   sa : in,  M x (K/128) float32
 *   b  : in,  N x K E4M3, 16-byte aligned   (Wgrad: X^T, N = in-channels)
 *   sb : in,  N x (K/128) float32 (one scale per row and group)
 *   c  : out, M x N, float32 or bfloat16, 16-byte aligned
 * Requires N % 128 == 0 and K % 128 == 0; M is arbitrary. M == 0 or N == 0
 * is a no-op; K == 0 writes zeros (a, sa, b, sb may then be NULL).
 */
FP8Q_API int fp8_gemm_rowscaled(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                void* c, int out_dtype, int64_t M, int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
