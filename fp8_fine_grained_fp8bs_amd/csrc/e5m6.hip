// e5m6.hip -- the 12-bit E5M6 format for cached activations (gfx950).
//
// [p1] para 3 (xn--9g3bo1gtkw0l8ubf92bgle.kr post wr_id=32373): a custom
// E5M6 format is used for some activations that are cached for the backward
// pass.  Layout taken: 12 bits, bit 11 sign, bits 10..6 exponent (bias 15),
// bits 5..0 mantissa, IEEE conventions (subnormals mant * 2^-20, exponent
// 31 for infinity); rows are packed, value i in bits 12 i .. 12 i + 11,
// little-endian (1.5 bytes per value).  Every E5M6 value is a bf16 value,
// so decoding to bf16 is exact and the backward re-quantization reads the
// decoded rows unchanged.
//
// Both kernels are streaming: a thread takes 8 consecutive values of a row
// (16 bytes of bf16, 12 bytes of E5M6), so a wave moves 1 KiB of bf16 and
// 768 contiguous bytes of E5M6 per instruction group.
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

// Nearest-even E5M6 code of a bf16 value (finite inputs; IEEE overflow to
// infinity).
__device__ __forceinline__ uint32_t e5m6_of_bf16(uint32_t b) {
  const uint32_t sign = (b >> 15) << 11;
  const uint32_t u = (b & 0x7fffu) << 16;           // |x| as FP32 bits
  uint32_t mag;
  if (u >= 0x477F8000u) {                           // >= 65280: halfway to 2^16 and beyond
    mag = 0x7C0u;
  } else if (u < 0x38800000u) {                     // below 2^-14: subnormal codes
    mag = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(u) * 0x1p20f));  // exact product, RNE
  } else {                                          // normal: round the mantissa to 6 bits
    const uint32_t r = u + 0xFFFFu + ((u >> 17) & 1u);
    mag = (r >> 17) - (112u << 6);                  // rebias 127 -> 15
  }
  return sign | mag;
}

// bf16 bit pattern of an E5M6 code (exact)
__device__ __forceinline__ uint32_t bf16_of_e5m6(uint32_t c) {
  const uint32_t sign = (c >> 11) << 15;
  const uint32_t e = (c >> 6) & 31u, m = c & 63u;
  uint32_t mag;
  if (e == 31u) mag = m ? 0x7FC0u : 0x7F80u;
  else if (e == 0u) mag = __float_as_uint(static_cast<float>(m) * 0x1p-20f) >> 16;  // exact
  else mag = ((e + 112u) << 7) | (m << 1);
  return sign | mag;
}

__global__ __launch_bounds__(256) void encode_e5m6_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                          uint8_t* __restrict__ y, int64_t ldy,
                                                          int64_t chunks, int64_t cpr) {
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = c / cpr, i = c - t * cpr;
    const uint4 v = load16_nt(x + t * ldx + i * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t code[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      code[2 * k] = e5m6_of_bf16(w[k] & 0xffffu);
      code[2 * k + 1] = e5m6_of_bf16(w[k] >> 16);
    }
    // 8 codes -> 96 bits, little-endian
    uint32_t* dst = reinterpret_cast<uint32_t*>(y + t * ldy + i * 12);
    dst[0] = code[0] | (code[1] << 12) | (code[2] << 24);
    dst[1] = (code[2] >> 8) | (code[3] << 4) | (code[4] << 16) | (code[5] << 28);
    dst[2] = (code[5] >> 4) | (code[6] << 8) | (code[7] << 20);
  }
}

__global__ __launch_bounds__(256) void decode_e5m6_kernel(const uint8_t* __restrict__ y, int64_t ldy,
                                                          uint16_t* __restrict__ x, int64_t ldx,
                                                          int64_t chunks, int64_t cpr) {
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = c / cpr, i = c - t * cpr;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(y + t * ldy + i * 12);
    // read once: non-temporal (41.5 against 58.5 us at 8192 x 7168 with the
    // caches full of dirty lines)
    const uint32_t d0 = __builtin_nontemporal_load(src), d1 = __builtin_nontemporal_load(src + 1),
                   d2 = __builtin_nontemporal_load(src + 2);
    const uint32_t code[8] = {d0 & 0xfffu,
                              (d0 >> 12) & 0xfffu,
                              (d0 >> 24) | ((d1 & 0xfu) << 8),
                              (d1 >> 4) & 0xfffu,
                              (d1 >> 16) & 0xfffu,
                              (d1 >> 28) | ((d2 & 0xffu) << 4),
                              (d2 >> 8) & 0xfffu,
                              d2 >> 20};
    uint4 o;
    o.x = bf16_of_e5m6(code[0]) | (bf16_of_e5m6(code[1]) << 16);
    o.y = bf16_of_e5m6(code[2]) | (bf16_of_e5m6(code[3]) << 16);
    o.z = bf16_of_e5m6(code[4]) | (bf16_of_e5m6(code[5]) << 16);
    o.w = bf16_of_e5m6(code[6]) | (bf16_of_e5m6(code[7]) << 16);
    *reinterpret_cast<uint4*>(x + t * ldx + i * 8) = o;
  }
}

int64_t stream_blocks(int64_t chunks) {
  int64_t blocks = (chunks + 255) / 256;
  return blocks > 16384 ? 16384 : blocks;   // more chunks in flight (4096: 5-10% slower cold)
}

}  // namespace

hipError_t launch_encode_e5m6(const uint16_t* x, int64_t T, int64_t C, int64_t ldx, uint8_t* y,
                              int64_t ldy, hipStream_t st) {
  const int64_t cpr = C / 8, chunks = T * cpr;
  hipLaunchKernelGGL(encode_e5m6_kernel, dim3(static_cast<unsigned>(stream_blocks(chunks))), dim3(256), 0,
                     st, x, ldx, y, ldy, chunks, cpr);
  return hipGetLastError();
}

hipError_t launch_decode_e5m6(const uint8_t* y, int64_t T, int64_t C, int64_t ldy, uint16_t* x,
                              int64_t ldx, hipStream_t st) {
  const int64_t cpr = C / 8, chunks = T * cpr;
  hipLaunchKernelGGL(decode_e5m6_kernel, dim3(static_cast<unsigned>(stream_blocks(chunks))), dim3(256), 0,
                     st, y, ldy, x, ldx, chunks, cpr);
  return hipGetLastError();
}

}  // namespace fp8bs
