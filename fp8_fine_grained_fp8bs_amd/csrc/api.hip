// api.hip -- the C ABI of libfp8bs: host-side argument checks and dispatch.
//
// Every check runs before the first HIP call, so a rejected call touches no
// device state.  Only after the checks pass is the current device queried
// (once per device, cached) and the kernel enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "fp8bs.h"
#include "fp8bs_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_dev_state[kMaxDevices];

// GEMM stride limits: a 256-row tile of codes or scales must span less than
// 4 GiB, so that 32-bit offsets from its first row reach every element.
constexpr int64_t kMaxCodeStride = int64_t(1) << 24;   // bytes per code row
constexpr int64_t kMaxScaleStride = int64_t(1) << 22;  // floats per scale row
constexpr int64_t kMaxRequantStride = int64_t(1) << 25;  // bytes per input row: requant, transpose

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fp8bs_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FP8BS_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return FP8BS_ERR_NO_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FP8BS_ERR_NO_DEVICE;
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? FP8BS_OK : FP8BS_ERR_NO_DEVICE;
}

fp8bs_status launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return FP8BS_ERR_LAUNCH;
  }
  return FP8BS_OK;
}

// Common checks of a row-major operand: stride and alignment.
fp8bs_status check_matrix(const void* p, int64_t cols, int64_t ld, int64_t elem_bytes) {
  if (p == nullptr) return FP8BS_ERR_INVALID_ARG;
  if (ld < cols) return FP8BS_ERR_INVALID_ARG;
  if (!aligned(p, 16) || (ld * elem_bytes) % 16 != 0) return FP8BS_ERR_MISALIGNED;
  return FP8BS_OK;
}

fp8bs_status check_scales(const float* p, int64_t cols, int64_t ld) {
  if (p == nullptr) return FP8BS_ERR_INVALID_ARG;
  if (ld < cols) return FP8BS_ERR_INVALID_ARG;
  if (!aligned(p, 4)) return FP8BS_ERR_MISALIGNED;
  return FP8BS_OK;
}

#define FP8BS_TRY(expr)                 \
  do {                                  \
    fp8bs_status _s = (expr);           \
    if (_s != FP8BS_OK) return _s;      \
  } while (0)

}  // namespace

extern "C" {

const char* fp8bs_status_string(fp8bs_status st) {
  switch (st) {
    case FP8BS_OK: return "FP8BS_OK";
    case FP8BS_ERR_INVALID_ARG: return "FP8BS_ERR_INVALID_ARG";
    case FP8BS_ERR_UNSUPPORTED_SHAPE: return "FP8BS_ERR_UNSUPPORTED_SHAPE";
    case FP8BS_ERR_MISALIGNED: return "FP8BS_ERR_MISALIGNED";
    case FP8BS_ERR_NO_DEVICE: return "FP8BS_ERR_NO_DEVICE";
    case FP8BS_ERR_LAUNCH: return "FP8BS_ERR_LAUNCH";
  }
  return "FP8BS_ERR_UNKNOWN";
}

int fp8bs_version(void) { return 100; }

fp8bs_status fp8bs_quant_act_1x128(const void* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                   void* stream) {
  if (M < 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (M == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(x, K, ldx, 2));
  FP8BS_TRY(check_matrix(q, K, ldq, 1));
  FP8BS_TRY(check_scales(s, K / 128, lds));
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_quant_act_1x128(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq,
                                                s, lds, static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_quant_act_w(const void* x, int64_t M, int64_t ldx, uint8_t* qx, int64_t ldqx,
                               float* sx, int64_t ldsx, const void* w, int64_t N, int64_t ldw,
                               uint8_t* qw, int64_t ldqw, float* sw, int64_t ldsw, int64_t K,
                               void* stream) {
  if (M < 0 || N < 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 && N == 0) return FP8BS_OK;
  if (M > 0) {
    FP8BS_TRY(check_matrix(x, K, ldx, 2));
    FP8BS_TRY(check_matrix(qx, K, ldqx, 1));
    FP8BS_TRY(check_scales(sx, K / 128, ldsx));
  }
  if (N > 0) {
    FP8BS_TRY(check_matrix(w, K, ldw, 2));
    FP8BS_TRY(check_matrix(qw, K, ldqw, 1));
    FP8BS_TRY(check_scales(sw, K / 128, ldsw));
  }
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_quant_act_w(static_cast<const uint16_t*>(x), M, ldx, qx, ldqx, sx, ldsx,
                                            static_cast<const uint16_t*>(w), N, ldw, qw, ldqw, sw, ldsw,
                                            K, static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_quant_w_128x128(const void* w, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                   void* stream) {
  if (N < 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (N == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(w, K, ldw, 2));
  FP8BS_TRY(check_matrix(q, K, ldq, 1));
  FP8BS_TRY(check_scales(s, K / 128, lds));
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_quant_w_128x128(static_cast<const uint16_t*>(w), N, K, ldw, q, ldq,
                                                s, lds, static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_quant_per_tensor(const void* x, int64_t n, uint8_t* q, float* s, void* stream) {
  if (n < 0) return FP8BS_ERR_INVALID_ARG;
  if (n % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (n == 0) return FP8BS_OK;
  if (x == nullptr || q == nullptr || s == nullptr) return FP8BS_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8BS_ERR_MISALIGNED;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_quant_per_tensor(static_cast<const uint16_t*>(x), n, q, s,
                                                 static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_cast_e4m3(const float* x, int64_t n, uint8_t* q, void* stream) {
  if (n < 0) return FP8BS_ERR_INVALID_ARG;
  if (n == 0) return FP8BS_OK;
  if (x == nullptr || q == nullptr) return FP8BS_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16)) return FP8BS_ERR_MISALIGNED;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_cast_e4m3(x, n, q, static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_encode_e5m6(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* y,
                               int64_t ldy, void* stream) {
  if (T < 0 || C <= 0) return FP8BS_ERR_INVALID_ARG;
  if (C % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(x, C, ldx, 2));
  FP8BS_TRY(check_matrix(y, C / 2 * 3, ldy, 1));
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_encode_e5m6(static_cast<const uint16_t*>(x), T, C, ldx, y, ldy,
                                            static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_decode_e5m6(const uint8_t* y, int64_t T, int64_t C, int64_t ldy, void* x,
                               int64_t ldx, void* stream) {
  if (T < 0 || C <= 0) return FP8BS_ERR_INVALID_ARG;
  if (C % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(y, C / 2 * 3, ldy, 1));
  FP8BS_TRY(check_matrix(x, C, ldx, 2));
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_decode_e5m6(y, T, C, ldy, static_cast<uint16_t*>(x), ldx,
                                            static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_swiglu_quant_1x128(const void* g, int64_t ldg, const void* u, int64_t ldu,
                                      int64_t T, int64_t I, uint8_t* q, int64_t ldq, float* s,
                                      int64_t lds, void* h, int64_t ldh, void* stream) {
  if (T < 0 || I <= 0) return FP8BS_ERR_INVALID_ARG;
  if (I % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if ((q == nullptr) != (s == nullptr)) return FP8BS_ERR_INVALID_ARG;
  if (q == nullptr && h == nullptr) return FP8BS_ERR_INVALID_ARG;
  if (T == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(g, I, ldg, 2));
  FP8BS_TRY(check_matrix(u, I, ldu, 2));
  if (q != nullptr) {
    FP8BS_TRY(check_matrix(q, I, ldq, 1));
    FP8BS_TRY(check_scales(s, I / 128, lds));
  }
  if (h != nullptr) FP8BS_TRY(check_matrix(h, I, ldh, 2));
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_swiglu_quant_1x128(static_cast<const uint16_t*>(g), ldg,
                                                   static_cast<const uint16_t*>(u), ldu, T, I, q, ldq, s,
                                                   lds, static_cast<uint16_t*>(h), ldh,
                                                   static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_requant_T_128x1(fp8bs_requant_src src, const void* in, const float* s_in,
                                   int64_t T, int64_t C, int64_t ld_in, int64_t lds_in,
                                   uint8_t* q_out, int64_t ld_out, float* s_out, int64_t lds_out,
                                   void* stream) {
  if (src != FP8BS_SRC_FP8_1x128 && src != FP8BS_SRC_BF16 && src != FP8BS_SRC_E5M6)
    return FP8BS_ERR_INVALID_ARG;
  if (T < 0 || C <= 0) return FP8BS_ERR_INVALID_ARG;
  if (C % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return FP8BS_OK;
  const bool codes = (src == FP8BS_SRC_FP8_1x128);
  // an input row: C codes, C bf16 values, or 1.5 C bytes of E5M6 (ld_in in bytes)
  const int64_t row_bytes = src == FP8BS_SRC_BF16 ? 2 * C : src == FP8BS_SRC_E5M6 ? C / 2 * 3 : C;
  const int64_t elem = src == FP8BS_SRC_BF16 ? 2 : 1;
  FP8BS_TRY(check_matrix(in, row_bytes / elem, ld_in, elem));
  if (codes) FP8BS_TRY(check_scales(s_in, C / 128, lds_in));
  FP8BS_TRY(check_matrix(q_out, T, ld_out, 1));
  FP8BS_TRY(check_scales(s_out, (T + 127) / 128, lds_out));
  // 128-token tiles are addressed with 32-bit offsets from their first row
  if (ld_in * elem >= kMaxRequantStride || (codes && lds_in >= kMaxScaleStride))
    return FP8BS_ERR_UNSUPPORTED_SHAPE;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_requant_T_128x1(static_cast<int>(src), in, s_in, T, C, ld_in, lds_in, q_out, ld_out,
                                                s_out, lds_out, static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_transpose_w_128x128(const uint8_t* q, int64_t N, int64_t K, int64_t ldq,
                                       const float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                                       float* st, int64_t ldst, void* stream) {
  if (N < 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (N % 128 != 0 || K % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (N == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(q, K, ldq, 1));
  FP8BS_TRY(check_scales(s, K / 128, lds));
  FP8BS_TRY(check_matrix(qt, N, ldqt, 1));
  FP8BS_TRY(check_scales(st, N / 128, ldst));
  // 128-row blocks are addressed with 32-bit offsets from their first row
  if (ldq >= kMaxRequantStride) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_transpose_w_128x128(q, N, K, ldq, s, lds, qt, ldqt, st, ldst,
                                                    static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_gemm(const uint8_t* a, const float* sa, int64_t lda, int64_t ldsa,
                        const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                        fp8bs_bscale bmode, void* d, int64_t ldd, fp8bs_out_dtype dt,
                        int64_t M, int64_t N, int64_t K, void* stream) {
  if (bmode != FP8BS_BSCALE_BLOCK_128x128 && bmode != FP8BS_BSCALE_ROW_1x128)
    return FP8BS_ERR_INVALID_ARG;
  if (dt != FP8BS_OUT_BF16 && dt != FP8BS_OUT_F32) return FP8BS_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(a, K, lda, 1));
  FP8BS_TRY(check_matrix(b, K, ldb, 1));
  FP8BS_TRY(check_scales(sa, K / 128, ldsa));
  FP8BS_TRY(check_scales(sb, K / 128, ldsb));
  FP8BS_TRY(check_matrix(d, N, ldd, dt == FP8BS_OUT_F32 ? 4 : 2));
  // tiles are addressed with 32-bit offsets from their first row
  if (lda >= kMaxCodeStride || ldb >= kMaxCodeStride || ldsa >= kMaxScaleStride ||
      ldsb >= kMaxScaleStride)
    return FP8BS_ERR_UNSUPPORTED_SHAPE;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_gemm(a, sa, lda, ldsa, b, sb, ldb, ldsb,
                                     bmode == FP8BS_BSCALE_ROW_1x128, d, ldd, nullptr, 0,
                                     dt == FP8BS_OUT_F32 ? 1 : 0, M, N, K,
                                     static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_gemm_quant_1x128(const uint8_t* a, const float* sa, int64_t lda, int64_t ldsa,
                                    const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                                    fp8bs_bscale bmode, uint8_t* q, int64_t ldq, float* s,
                                    int64_t lds, int64_t M, int64_t N, int64_t K, void* stream) {
  if (bmode != FP8BS_BSCALE_BLOCK_128x128 && bmode != FP8BS_BSCALE_ROW_1x128)
    return FP8BS_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (K % 128 != 0 || N % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(a, K, lda, 1));
  FP8BS_TRY(check_matrix(b, K, ldb, 1));
  FP8BS_TRY(check_scales(sa, K / 128, ldsa));
  FP8BS_TRY(check_scales(sb, K / 128, ldsb));
  FP8BS_TRY(check_matrix(q, N, ldq, 1));
  FP8BS_TRY(check_scales(s, N / 128, lds));
  if (lda >= kMaxCodeStride || ldb >= kMaxCodeStride || ldsa >= kMaxScaleStride ||
      ldsb >= kMaxScaleStride)
    return FP8BS_ERR_UNSUPPORTED_SHAPE;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_gemm(a, sa, lda, ldsa, b, sb, ldb, ldsb,
                                     bmode == FP8BS_BSCALE_ROW_1x128, q, ldq, s, lds, 2, M, N, K,
                                     static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_gemm_bf16a(const void* x, int64_t ldx, uint8_t* qx, int64_t ldqx, float* sx,
                              int64_t ldsx, const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                              void* d, int64_t ldd, fp8bs_out_dtype dt, int64_t M, int64_t N, int64_t K,
                              void* stream) {
  if (dt != FP8BS_OUT_BF16 && dt != FP8BS_OUT_F32) return FP8BS_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if ((qx == nullptr) != (sx == nullptr)) return FP8BS_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(x, K, ldx, 2));
  FP8BS_TRY(check_matrix(b, K, ldb, 1));
  FP8BS_TRY(check_scales(sb, K / 128, ldsb));
  FP8BS_TRY(check_matrix(d, N, ldd, dt == FP8BS_OUT_F32 ? 4 : 2));
  if (qx != nullptr) {
    FP8BS_TRY(check_matrix(qx, K, ldqx, 1));
    FP8BS_TRY(check_scales(sx, K / 128, ldsx));
  }
  // 64-row tiles of bf16 A and 256-row tiles of codes are addressed with
  // 32-bit offsets from their first row
  if (ldx >= kMaxCodeStride / 2 || ldb >= kMaxCodeStride || ldsb >= kMaxScaleStride)
    return FP8BS_ERR_UNSUPPORTED_SHAPE;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_gemm_bf16a(static_cast<const uint16_t*>(x), ldx, qx, ldqx, sx, ldsx, b, sb,
                                           ldb, ldsb, d, ldd, dt == FP8BS_OUT_F32, M, N, K,
                                           static_cast<hipStream_t>(stream)));
}

fp8bs_status fp8bs_grouped_gemm(const uint8_t* a, const float* sa, int64_t ldsa,
                                const uint8_t* b, const float* sb,
                                const int32_t* offsets, int32_t E, int64_t M_total,
                                void* d, fp8bs_out_dtype dt, int64_t N, int64_t K,
                                void* stream) {
  if (dt != FP8BS_OUT_BF16 && dt != FP8BS_OUT_F32) return FP8BS_ERR_INVALID_ARG;
  if (E < 1 || M_total < 0 || N <= 0 || K <= 0) return FP8BS_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  if (offsets == nullptr || b == nullptr || sb == nullptr) return FP8BS_ERR_INVALID_ARG;
  if (!aligned(offsets, 4) || !aligned(sb, 4) || !aligned(b, 16)) return FP8BS_ERR_MISALIGNED;
  if (M_total == 0) return FP8BS_OK;
  FP8BS_TRY(check_matrix(a, K, K, 1));
  FP8BS_TRY(check_scales(sa, K / 128, ldsa));
  FP8BS_TRY(check_matrix(d, N, N, dt == FP8BS_OUT_F32 ? 4 : 2));
  if (K >= kMaxCodeStride || ldsa >= kMaxScaleStride) return FP8BS_ERR_UNSUPPORTED_SHAPE;
  FP8BS_TRY(check_device());
  return launched(fp8bs::launch_grouped_gemm(a, sa, ldsa, b, sb, offsets, E, M_total, d,
                                             dt == FP8BS_OUT_F32, N, K,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
