// C ABI of the fp8q library: host-side argument checks, then kernel launches.
// Every check runs before the first HIP call, so a rejected call touches no
// device state and can be exercised without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/fp8q.h"

namespace fp8q {
hipError_t launch_quant_act_1x128(const void* x, int64_t M, int64_t K, uint8_t* q, float* sa,
                                  bool nontemporal, hipStream_t stream);
hipError_t launch_quant_weight_128x128(const void* w, int64_t N, int64_t K, uint8_t* q, float* sb,
                                       hipStream_t stream);
hipError_t launch_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                   const float* sb, void* c, bool bf16_out, int64_t M, int64_t N,
                                   int64_t K, hipStream_t stream);
hipError_t launch_gemm_grouped(const uint8_t* a, const float* sa, const uint8_t* b,
                               const float* sb, void* c, bool bf16_out, const int32_t* m_offsets,
                               int64_t G, int64_t M_total, int64_t N, int64_t K,
                               hipStream_t stream);
int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_blockscaled_ws(const uint8_t* a, const float* sa, const uint8_t* b,
                                      const float* sb, void* c, bool bf16_out, int64_t M,
                                      int64_t N, int64_t K, float* ws, hipStream_t stream);
hipError_t launch_gemm_rowscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                 const float* sb_rows, void* c, bool bf16_out, int64_t M, int64_t N,
                                 int64_t K, hipStream_t stream);
int64_t static_scratch_bytes();
hipError_t launch_gemm_blockscaled_static(const uint8_t* a, const float* sa, const uint8_t* b,
                                          const float* sb, void* c, bool bf16_out, int64_t M,
                                          int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_gemm_quant_a(const void* a, const uint8_t* b, const float* sb, void* c,
                               bool bf16_out, int64_t M, int64_t N, int64_t K, uint8_t* qa,
                               float* sa, hipStream_t stream);
hipError_t launch_quant_act_128x1(const void* x, int64_t M, int64_t K, uint8_t* qt, float* st,
                                  hipStream_t stream);
hipError_t launch_norm_quant_act_1x128(const void* x, const void* gamma, const void* beta,
                                       float eps, bool centred, int64_t M, int64_t K, uint8_t* q,
                                       float* sa, hipStream_t stream);
int64_t dispatch_workspace_bytes(int64_t slots, int64_t G);
hipError_t launch_moe_dispatch(const void* x, const int32_t* ids, int64_t T, int64_t K, int64_t k,
                               int64_t G, uint8_t* q, float* sa, int32_t* m_offsets,
                               int32_t* row_of_slot, void* workspace, hipStream_t stream);
hipError_t launch_quant_act_dual(const void* x, int64_t M, int64_t K, uint8_t* q, float* sa,
                                 uint8_t* qt, float* st, hipStream_t stream);
hipError_t launch_requant_1x128_to_128x1(const uint8_t* q, const float* sa, int64_t M, int64_t K,
                                         uint8_t* qt, float* st, hipStream_t stream);
hipError_t launch_transpose_weight_128x128(const uint8_t* q, const float* sb, int64_t N, int64_t K,
                                           uint8_t* qt, float* sbt, hipStream_t stream);
}  // namespace fp8q

namespace {

constexpr int64_t kGroup = 128;
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;  // kernels index rows/cols with int32
// GEMM operand tiles (up to 256 rows of K bytes) are addressed with 32-bit
// offsets through buffer descriptors
constexpr int64_t kMaxK = int64_t(1) << 23;
constexpr int64_t kMaxExperts = 1024;  // dispatch: one scan thread per expert
// the fused normalization keeps a row in one wavefront's registers
constexpr int64_t kNormMaxK = 16384;
constexpr int kMaxDevices = 64;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// 0 = unknown, 1 = gfx950, 2 = other; one slot per device ordinal.
std::atomic<int> g_device_kind[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8Q_ERR_NO_DEVICE;
  if (dev >= kMaxDevices) return FP8Q_ERR_NO_DEVICE;
  int kind = g_device_kind[dev].load(std::memory_order_relaxed);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8Q_ERR_NO_DEVICE;
    kind = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_kind[dev].store(kind, std::memory_order_relaxed);
  }
  return kind == 1 ? FP8Q_OK : FP8Q_ERR_NO_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_LAUNCH; }

int check_gemm_common(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                      const void* c, int out_dtype, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return FP8Q_ERR_SHAPE;
  if (N % kGroup || K % kGroup) return FP8Q_ERR_SHAPE;
  if (out_dtype != FP8Q_OUT_F32 && out_dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxK) return FP8Q_ERR_TOO_LARGE;
  if ((M + 127) / 128 * (N / 128) > kMaxDim) return FP8Q_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return -1;  // valid no-op
  if (!c) return FP8Q_ERR_NULL;
  if (K > 0 && (!a || !sa || !b || !sb)) return FP8Q_ERR_NULL;  // K == 0 reads no operand
  if (!aligned(c, 16)) return FP8Q_ERR_ALIGN;
  if (K > 0 && (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4)))
    return FP8Q_ERR_ALIGN;
  return FP8Q_OK;
}

// worst-case m_offsets[G] of the MoE dispatch (every expert padded by 127
// rows), rounded up to a multiple of 128 so that it is a valid M_total for
// the grouped GEMM
int64_t dispatch_max_rows(int64_t T, int64_t topk, int64_t G) {
  return (T * topk + (kGroup - 1) * G + kGroup - 1) / kGroup * kGroup;
}

// Checks shared by the three 128 x 128 tile re-tiling calls (R x C -> C x R).
int check_retile(const void* in, const float* in_s, bool need_in_s, int64_t R, int64_t C,
                 const uint8_t* out, const float* out_s) {
  if (R < 0 || C < 0 || R % kGroup || C % kGroup) return FP8Q_ERR_SHAPE;
  if (R > kMaxDim || C > kMaxDim || C / kGroup > 65535) return FP8Q_ERR_TOO_LARGE;
  if (R == 0 || C == 0) return -1;  // valid no-op
  if (!in || !out || !out_s || (need_in_s && !in_s)) return FP8Q_ERR_NULL;
  if (!aligned(in, 16) || !aligned(out, 16) || !aligned(out_s, 4)) return FP8Q_ERR_ALIGN;
  if (need_in_s && !aligned(in_s, 4)) return FP8Q_ERR_ALIGN;
  return FP8Q_OK;
}

}  // namespace

extern "C" {

int fp8q_version(void) { return 202; }

const char* fp8q_status_string(int status) {
  switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_ERR_NULL: return "a required pointer is NULL";
    case FP8Q_ERR_SHAPE: return "invalid shape (negative size, K or N not a multiple of 128, or G < 1)";
    case FP8Q_ERR_ALIGN: return "misaligned pointer (16 bytes for data, 4 bytes for scales)";
    case FP8Q_ERR_DTYPE: return "unknown output dtype";
    case FP8Q_ERR_LAUNCH: return "kernel launch failed";
    case FP8Q_ERR_NO_DEVICE: return "no gfx950 device is current";
    case FP8Q_ERR_TOO_LARGE: return "size exceeds the kernels' 32-bit indexing";
    case FP8Q_ERR_SCRATCH: return "the split-K partials exceed the library's static scratch (8 MiB)";
    default: return "unknown status";
  }
}

static int quant_act_1x128(const void* x_bf16, int64_t M, int64_t K, uint8_t* q, float* sa,
                           bool nontemporal, void* stream) {
  if (M < 0 || K < 0 || K % kGroup) return FP8Q_ERR_SHAPE;
  if (M > kMaxDim || K > kMaxDim || M * (K / kGroup) > (kMaxDim / 16)) return FP8Q_ERR_TOO_LARGE;
  if (M == 0 || K == 0) return FP8Q_OK;
  if (!x_bf16 || !q || !sa) return FP8Q_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(sa, 4)) return FP8Q_ERR_ALIGN;
  if (int s = check_device()) return s;
  return launched(fp8q::launch_quant_act_1x128(x_bf16, M, K, q, sa, nontemporal, (hipStream_t)stream));
}

int fp8q_quant_act_1x128(const void* x_bf16, int64_t M, int64_t K, uint8_t* q, float* sa,
                         void* stream) {
  return quant_act_1x128(x_bf16, M, K, q, sa, false, stream);
}

int fp8q_quant_act_1x128_nt(const void* x_bf16, int64_t M, int64_t K, uint8_t* q, float* sa,
                            void* stream) {
  return quant_act_1x128(x_bf16, M, K, q, sa, true, stream);
}

int fp8q_quant_weight_128x128(const void* w_bf16, int64_t N, int64_t K, uint8_t* q, float* sb,
                              void* stream) {
  if (N < 0 || K < 0 || N % kGroup || K % kGroup) return FP8Q_ERR_SHAPE;
  if (N / kGroup > 65535 || K > kMaxDim) return FP8Q_ERR_TOO_LARGE;
  if (N == 0 || K == 0) return FP8Q_OK;
  if (!w_bf16 || !q || !sb) return FP8Q_ERR_NULL;
  if (!aligned(w_bf16, 16) || !aligned(q, 16) || !aligned(sb, 4)) return FP8Q_ERR_ALIGN;
  if (int s = check_device()) return s;
  return launched(fp8q::launch_quant_weight_128x128(w_bf16, N, K, q, sb, (hipStream_t)stream));
}

int fp8_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                         void* c, int out_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  int s = check_gemm_common(a, sa, b, sb, c, out_dtype, M, N, K);
  if (s == -1) return FP8Q_OK;
  if (s) return s;
  if ((s = check_device())) return s;
  return launched(fp8q::launch_gemm_blockscaled(a, sa, b, sb, c, out_dtype == FP8Q_OUT_BF16, M, N,
                                                K, (hipStream_t)stream));
}

int fp8_gemm_blockscaled_bf16a(const void* a, const uint8_t* b, const float* sb, void* c,
                               int out_dtype, int64_t M, int64_t N, int64_t K, uint8_t* qa, float* sa,
                               void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP8Q_ERR_SHAPE;
  if (N % kGroup || K % kGroup) return FP8Q_ERR_SHAPE;
  if (out_dtype != FP8Q_OUT_F32 && out_dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxK) return FP8Q_ERR_TOO_LARGE;
  if ((M + 127) / 128 * ((N + 255) / 256) > kMaxDim) return FP8Q_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return FP8Q_OK;  // valid no-op (no outputs written)
  if (!c) return FP8Q_ERR_NULL;
  if ((qa == nullptr) != (sa == nullptr)) return FP8Q_ERR_NULL;  // both outputs or neither
  if (K > 0 && (!a || !b || !sb)) return FP8Q_ERR_NULL;         // K == 0 reads no operand
  if (!aligned(c, 16)) return FP8Q_ERR_ALIGN;
  if (K > 0 && (!aligned(a, 16) || !aligned(b, 16) || !aligned(sb, 4))) return FP8Q_ERR_ALIGN;
  if (qa && (!aligned(qa, 16) || !aligned(sa, 4))) return FP8Q_ERR_ALIGN;
  int s;
  if ((s = check_device())) return s;
  return launched(fp8q::launch_gemm_quant_a(a, b, sb, c, out_dtype == FP8Q_OUT_BF16, M, N, K,
                                            K > 0 ? qa : nullptr, K > 0 ? sa : nullptr,
                                            (hipStream_t)stream));
}

int64_t fp8_gemm_blockscaled_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || N % kGroup || K % kGroup) return -1;
  if (M > kMaxDim || N > kMaxDim || K > kMaxK) return -1;
  return fp8q::splitk_workspace_bytes(M, N, K);
}

int fp8_gemm_blockscaled_ws(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                            void* c, int out_dtype, int64_t M, int64_t N, int64_t K,
                            void* workspace, int64_t workspace_bytes, void* stream) {
  int s = check_gemm_common(a, sa, b, sb, c, out_dtype, M, N, K);
  if (s == -1) return FP8Q_OK;
  if (s) return s;
  const int64_t need = fp8q::splitk_workspace_bytes(M, N, K);
  if (need > 0) {
    if (!workspace) return FP8Q_ERR_NULL;
    if (workspace_bytes < need) return FP8Q_ERR_SHAPE;
    if (!aligned(workspace, 16)) return FP8Q_ERR_ALIGN;
  }
  if ((s = check_device())) return s;
  return launched(fp8q::launch_gemm_blockscaled_ws(a, sa, b, sb, c, out_dtype == FP8Q_OUT_BF16, M, N,
                                                   K, need > 0 ? (float*)workspace : nullptr,
                                                   (hipStream_t)stream));
}

int fp8_gemm_blockscaled_noalloc(const uint8_t* a, const float* sa, const uint8_t* b,
                                 const float* sb, void* c, int out_dtype, int64_t M, int64_t N,
                                 int64_t K, void* stream) {
  int s = check_gemm_common(a, sa, b, sb, c, out_dtype, M, N, K);
  if (s == -1) return FP8Q_OK;
  if (s) return s;
  if (fp8q::splitk_workspace_bytes(M, N, K) > fp8q::static_scratch_bytes()) return FP8Q_ERR_SCRATCH;
  if ((s = check_device())) return s;
  return launched(fp8q::launch_gemm_blockscaled_static(a, sa, b, sb, c, out_dtype == FP8Q_OUT_BF16,
                                                       M, N, K, (hipStream_t)stream));
}

int fp8_gemm_grouped(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                     void* c, int out_dtype, const int32_t* m_offsets, int64_t G, int64_t M_total,
                     int64_t N, int64_t K, void* stream) {
  if (G < 1) return FP8Q_ERR_SHAPE;
  if (M_total % kGroup) return FP8Q_ERR_SHAPE;
  if (G > kMaxDim || G * N > kMaxDim) return FP8Q_ERR_TOO_LARGE;
  int s = check_gemm_common(a, sa, b, sb, c, out_dtype, M_total, N, K);
  if (s == -1) return FP8Q_OK;
  if (s) return s;
  if (!m_offsets) return FP8Q_ERR_NULL;
  if (!aligned(m_offsets, 4)) return FP8Q_ERR_ALIGN;
  if ((s = check_device())) return s;
  return launched(fp8q::launch_gemm_grouped(a, sa, b, sb, c, out_dtype == FP8Q_OUT_BF16,
                                            m_offsets, G, M_total, N, K, (hipStream_t)stream));
}

int fp8q_quant_act_128x1(const void* x_bf16, int64_t M, int64_t K, uint8_t* qt, float* st,
                         void* stream) {
  int s = check_retile(x_bf16, nullptr, false, M, K, qt, st);
  if (s == -1) return FP8Q_OK;
  if (s || (s = check_device())) return s;
  return launched(fp8q::launch_quant_act_128x1(x_bf16, M, K, qt, st, (hipStream_t)stream));
}

int64_t fp8q_moe_dispatch_workspace_bytes(int64_t T, int64_t topk, int64_t G) {
  if (T < 0 || topk < 1 || G < 1 || G > kMaxExperts) return -1;
  if (T > kMaxDim / topk) return -1;
  return fp8q::dispatch_workspace_bytes(T * topk, G);
}

int64_t fp8q_moe_dispatch_max_rows(int64_t T, int64_t topk, int64_t G) {
  if (T < 0 || topk < 1 || G < 1 || G > kMaxExperts) return -1;
  if (T > kMaxDim / topk) return -1;
  return dispatch_max_rows(T, topk, G);
}

int fp8q_moe_dispatch_1x128(const void* x_bf16, const int32_t* topk_ids, int64_t T, int64_t K,
                            int64_t topk, int64_t G, uint8_t* q, float* sa, int64_t M_cap,
                            int32_t* m_offsets, int32_t* row_of_slot, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  if (T < 0 || K < 0 || K % kGroup || topk < 1 || G < 1) return FP8Q_ERR_SHAPE;
  if (G > kMaxExperts || K > kMaxDim || T > kMaxDim / topk) return FP8Q_ERR_TOO_LARGE;
  const int64_t need_rows = dispatch_max_rows(T, topk, G);
  if (need_rows > kMaxDim || T > kMaxDim / 4) return FP8Q_ERR_TOO_LARGE;
  if (M_cap < need_rows) return FP8Q_ERR_SHAPE;  // outputs too small for the worst-case padding
  if (!m_offsets || !workspace) return FP8Q_ERR_NULL;
  if (T > 0 && (!topk_ids || !row_of_slot)) return FP8Q_ERR_NULL;
  if (K > 0 && (!q || !sa || (T > 0 && !x_bf16))) return FP8Q_ERR_NULL;
  if (workspace_bytes < fp8q::dispatch_workspace_bytes(T * topk, G)) return FP8Q_ERR_SHAPE;
  if (!aligned(m_offsets, 4) || !aligned(workspace, 4)) return FP8Q_ERR_ALIGN;
  if (T > 0 && (!aligned(topk_ids, 4) || !aligned(row_of_slot, 4))) return FP8Q_ERR_ALIGN;
  if (K > 0 && (!aligned(q, 16) || !aligned(sa, 4) || (T > 0 && !aligned(x_bf16, 16))))
    return FP8Q_ERR_ALIGN;
  if (int s = check_device()) return s;
  return launched(fp8q::launch_moe_dispatch(x_bf16, topk_ids, T, K, topk, G, q, sa, m_offsets,
                                            row_of_slot, workspace, (hipStream_t)stream));
}

int fp8q_norm_quant_act_1x128(const void* x_bf16, const void* gamma_bf16, const void* beta_bf16,
                              float eps, int centred, int64_t M, int64_t K, uint8_t* q, float* sa,
                              void* stream) {
  if (M < 0 || K < 0 || K % kGroup) return FP8Q_ERR_SHAPE;
  if (centred != 0 && centred != 1) return FP8Q_ERR_SHAPE;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return FP8Q_ERR_SHAPE;  // NaN, negative or infinite
  if (M > kMaxDim || K > kNormMaxK) return FP8Q_ERR_TOO_LARGE;
  if (M == 0 || K == 0) return FP8Q_OK;
  if (!x_bf16 || !gamma_bf16 || !q || !sa || (centred && !beta_bf16)) return FP8Q_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(gamma_bf16, 16) || !aligned(q, 16) || !aligned(sa, 4))
    return FP8Q_ERR_ALIGN;
  if (centred && !aligned(beta_bf16, 16)) return FP8Q_ERR_ALIGN;
  if (int s = check_device()) return s;
  return launched(fp8q::launch_norm_quant_act_1x128(x_bf16, gamma_bf16, beta_bf16, eps,
                                                    centred == 1, M, K, q, sa,
                                                    (hipStream_t)stream));
}

int fp8q_quant_act_1x128_128x1(const void* x_bf16, int64_t M, int64_t K, uint8_t* q, float* sa,
                               uint8_t* qt, float* st, void* stream) {
  int s = check_retile(x_bf16, nullptr, false, M, K, qt, st);
  if (s == -1) return FP8Q_OK;
  if (s) return s;
  if (!q || !sa) return FP8Q_ERR_NULL;
  if (!aligned(q, 16) || !aligned(sa, 4)) return FP8Q_ERR_ALIGN;
  if ((s = check_device())) return s;
  return launched(fp8q::launch_quant_act_dual(x_bf16, M, K, q, sa, qt, st, (hipStream_t)stream));
}

int fp8q_requant_1x128_to_128x1(const uint8_t* q, const float* sa, int64_t M, int64_t K,
                                uint8_t* qt, float* st, void* stream) {
  int s = check_retile(q, sa, true, M, K, qt, st);
  if (s == -1) return FP8Q_OK;
  if (s || (s = check_device())) return s;
  return launched(fp8q::launch_requant_1x128_to_128x1(q, sa, M, K, qt, st, (hipStream_t)stream));
}

int fp8q_transpose_weight_128x128(const uint8_t* q, const float* sb, int64_t N, int64_t K,
                                  uint8_t* qt, float* sbt, void* stream) {
  int s = check_retile(q, sb, true, N, K, qt, sbt);
  if (s == -1) return FP8Q_OK;
  if (s || (s = check_device())) return s;
  return launched(fp8q::launch_transpose_weight_128x128(q, sb, N, K, qt, sbt, (hipStream_t)stream));
}

int fp8_gemm_rowscaled(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                       void* c, int out_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  int s = check_gemm_common(a, sa, b, sb, c, out_dtype, M, N, K);
  if (s == -1) return FP8Q_OK;
  if (s) return s;
  if ((s = check_device())) return s;
  return launched(fp8q::launch_gemm_rowscaled(a, sa, b, sb, c, out_dtype == FP8Q_OUT_BF16, M, N, K,
                                              (hipStream_t)stream));
}

}  // extern "C"
