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
// 768 contiguous bytes of E5M6 per instruction group.  Both convert by way
// of FP16, whose encoding has the E5M6 fields in its upper 12 bits, with
// packed 16-bit integer operations: a few instructions per value and no
// branch per value (decoding the fields one value at a time with branches
// took about 16, enough to hold these kernels below the HBM rate).
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

// Codes of two bf16 values (value 0 in the lower half of w) by way of FP16:
// the E5M6 code of a value is its FP16 encoding rounded to the upper 12 bits
// (sign, 5-bit exponent with bias 15, subnormals and infinity alike), so one
// packed FP32 -> FP16 conversion (round to nearest even, overflow to
// infinity from 65520) followed by a 16-bit round to nearest even at bit 4
// gives both codes; the carry of that rounding moves a mantissa of all ones
// into the next exponent (and 65280 .. 65519 into infinity) as it should.
// The conversion to FP16 is exact for |x| >= 2^-17 and for 0; below that
// the two roundings could meet at a tie of the second, so `tiny` is set for
// such values (0 < |x| < 2^-17) and the caller takes e5m6_of_bf16 for them.
// Result: code 0 in bits 0..11, code 1 in bits 12..23.
__device__ __forceinline__ uint32_t e5m6x2_of_bf16x2(uint32_t w, u16x2_t& tiny_min) {
  const f32x2_t x = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  const u16x2_t h = __builtin_bit_cast(u16x2_t, __builtin_convertvector(x, f16x2_t));
  // |h| - 1 wraps 0 to 0xFFFF: the min over a thread's values is below
  // 0x7F exactly when one of them is tiny
  tiny_min = __builtin_elementwise_min(tiny_min, (h & u16x2_t{0x7fff, 0x7fff}) - u16x2_t{1, 1});
  const u16x2_t r = (h + ((h >> u16x2_t{4, 4}) & u16x2_t{1, 1}) + u16x2_t{7, 7}) >> u16x2_t{4, 4};
  const uint32_t q = __builtin_bit_cast(uint32_t, r);   // code 0 at bits 0..11, code 1 at 16..27
  return __builtin_amdgcn_ubfe(q, 0, 12) | ((q >> 4) & 0xfff000u);
}

// A thread's chunk of a row: 8 values (16 bytes of bf16, 12 of E5M6).  The
// grid walks the T x C/8 chunks row by row, each thread stepping by the
// grid's size without a division per step.
struct ChunkWalk {
  int64_t t, i;   // row, chunk in the row
  __device__ ChunkWalk(int64_t cpr) {
    const uint32_t c0 = blockIdx.x * 256u + threadIdx.x;   // < 2^32: the grid is capped
    t = c0 / static_cast<uint64_t>(cpr);
    i = c0 - t * cpr;
  }
  __device__ void next(int64_t q_step, int64_t r_step, int64_t cpr) {
    t += q_step;
    i += r_step;
    if (i >= cpr) {
      i -= cpr;
      ++t;
    }
  }
};

__global__ __launch_bounds__(256) void encode_e5m6_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                          uint8_t* __restrict__ y, int64_t ldy, int64_t T,
                                                          int64_t cpr, int64_t q_step, int64_t r_step) {
  for (ChunkWalk c(cpr); c.t < T; c.next(q_step, r_step, cpr)) {
    const uint4 v = load16_nt(x + c.t * ldx + c.i * 8);
    u16x2_t tiny = {0xffff, 0xffff};
    uint32_t p[4] = {e5m6x2_of_bf16x2(v.x, tiny), e5m6x2_of_bf16x2(v.y, tiny), e5m6x2_of_bf16x2(v.z, tiny),
                     e5m6x2_of_bf16x2(v.w, tiny)};
    if (__builtin_expect(__builtin_elementwise_min(tiny.x, tiny.y) < 0x7f, 0)) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = e5m6_of_bf16(w[k] & 0xffffu) | (e5m6_of_bf16(w[k] >> 16) << 12);
    }
    // four 24-bit pairs -> 96 bits, little-endian (byte moves)
    uint32_t* dst = reinterpret_cast<uint32_t*>(y + c.t * ldy + c.i * 12);
    dst[0] = __builtin_amdgcn_perm(p[1], p[0], 0x04020100u);
    dst[1] = __builtin_amdgcn_perm(p[2], p[1], 0x05040201u);
    dst[2] = __builtin_amdgcn_perm(p[3], p[2], 0x06050402u);
  }
}

__global__ __launch_bounds__(256) void decode_e5m6_kernel(const uint8_t* __restrict__ y, int64_t ldy,
                                                          uint16_t* __restrict__ x, int64_t ldx, int64_t T,
                                                          int64_t cpr, int64_t q_step, int64_t r_step) {
  for (ChunkWalk c(cpr); c.t < T; c.next(q_step, r_step, cpr)) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(y + c.t * ldy + c.i * 12);
    // read once: non-temporal (41.5 against 58.5 us at 8192 x 7168 with the
    // caches full of dirty lines)
    const uint32_t d0 = __builtin_nontemporal_load(src), d1 = __builtin_nontemporal_load(src + 1),
                   d2 = __builtin_nontemporal_load(src + 2);
    uint4 o = bf16x8_of_e5m6x8_f16(d0, d1, d2);
    o = make_uint4(canonical_nan_bf16x2(o.x), canonical_nan_bf16x2(o.y), canonical_nan_bf16x2(o.z),
                   canonical_nan_bf16x2(o.w));
    *reinterpret_cast<uint4*>(x + c.t * ldx + c.i * 8) = o;
  }
}

int64_t stream_blocks(int64_t chunks) {
  int64_t blocks = (chunks + 255) / 256;
  return blocks > 16384 ? 16384 : blocks;   // more chunks in flight (4096: 5-10% slower cold)
}

}  // namespace

hipError_t launch_encode_e5m6(const uint16_t* x, int64_t T, int64_t C, int64_t ldx, uint8_t* y,
                              int64_t ldy, hipStream_t st) {
  const int64_t cpr = C / 8, blocks = stream_blocks(T * cpr), step = blocks * 256;
  hipLaunchKernelGGL(encode_e5m6_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, x, ldx, y, ldy,
                     T, cpr, step / cpr, step % cpr);
  return hipGetLastError();
}

hipError_t launch_decode_e5m6(const uint8_t* y, int64_t T, int64_t C, int64_t ldy, uint16_t* x,
                              int64_t ldx, hipStream_t st) {
  const int64_t cpr = C / 8, blocks = stream_blocks(T * cpr), step = blocks * 256;
  hipLaunchKernelGGL(decode_e5m6_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, y, ldy, x, ldx,
                     T, cpr, step / cpr, step % cpr);
  return hipGetLastError();
}

}  // namespace fp8bs
