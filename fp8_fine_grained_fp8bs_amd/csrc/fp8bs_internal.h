// fp8bs_internal.h -- launchers behind the C ABI (arguments already checked).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

hipError_t launch_quant_act_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                  hipStream_t st);

hipError_t launch_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                  hipStream_t st);

hipError_t launch_quant_act_w(const uint16_t* x, int64_t M, int64_t ldx, uint8_t* qx, int64_t ldqx,
                              float* sx, int64_t ldsx, const uint16_t* w, int64_t N, int64_t ldw,
                              uint8_t* qw, int64_t ldqw, float* sw, int64_t ldsw, int64_t K,
                              hipStream_t st);

hipError_t launch_cast_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t st);

hipError_t launch_swiglu_quant_1x128(const uint16_t* g, int64_t ldg, const uint16_t* u, int64_t ldu,
                                     int64_t T, int64_t I, uint8_t* q, int64_t ldq, float* s,
                                     int64_t lds, uint16_t* h, int64_t ldh, hipStream_t st);

hipError_t launch_quant_per_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* s,
                                   hipStream_t st);

hipError_t launch_encode_e5m6(const uint16_t* x, int64_t T, int64_t C, int64_t ldx, uint8_t* y,
                              int64_t ldy, hipStream_t st);

hipError_t launch_decode_e5m6(const uint8_t* y, int64_t T, int64_t C, int64_t ldy, uint16_t* x,
                              int64_t ldx, hipStream_t st);

// src: 0 E4M3 codes with 1x128 scales, 1 bf16, 2 packed E5M6
hipError_t launch_requant_T_128x1(int src, const void* in, const float* s_in,
                                  int64_t T, int64_t C, int64_t ld_in, int64_t lds_in,
                                  uint8_t* q_out, int64_t ld_out, float* s_out,
                                  int64_t lds_out, hipStream_t st);

hipError_t launch_transpose_w_128x128(const uint8_t* q, int64_t N, int64_t K, int64_t ldq,
                                      const float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                                      float* st, int64_t ldst, hipStream_t stream);

hipError_t launch_gemm(const uint8_t* a, const float* sa, int64_t lda, int64_t ldsa,
                       const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                       bool bscale_row, void* d, int64_t ldd, float* s_out, int64_t lds_out,
                       int out, int64_t M, int64_t N, int64_t K, hipStream_t st);

hipError_t launch_gemm_bf16a(const uint16_t* x, int64_t ldx, uint8_t* qx, int64_t ldqx, float* sx,
                             int64_t ldsx, const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                             void* d, int64_t ldd, bool out_f32, int64_t M, int64_t N, int64_t K,
                             hipStream_t st);

hipError_t launch_grouped_gemm(const uint8_t* a, const float* sa, int64_t ldsa,
                               const uint8_t* b, const float* sb, const int32_t* offsets,
                               int32_t E, int64_t M_total, void* d, bool out_f32,
                               int64_t N, int64_t K, hipStream_t st);

}  // namespace fp8bs
