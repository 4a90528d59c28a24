// fp8bs_device.h -- device helpers shared by the libfp8bs kernels (gfx950).
//
// E4M3 encoding that is bit-exact with "nearest-even E4M3 of the exact
// quotient x / s, saturated to +-448" at the cost of two multiplies and one
// hardware conversion per value:
//
//   With r ~ 1/s, the two products y_lo = x * r(1 - 2^-20) and
//   y_hi = x * r(1 + 2^-20) bracket the exact quotient q = x / s (the margin
//   2^-20 exceeds the error of r, 2^-23, plus the rounding of both products).
//   v_cvt_pk_fp8_f32 rounds to nearest-even, is monotone, keeps the sign of
//   zero and maps (448, 464] to 448 (checked exhaustively on gfx950 over
//   every float with |f| <= 448 and the boundary values above it), so when
//   y_lo and y_hi convert to the same code that code is the code of q.
//   Otherwise exactly one E4M3 rounding midpoint mu lies between them and the
//   sign of |x| - mu * s, formed exactly by one fma, picks the side (a zero
//   picks the even code).  The exactness of that fma needs s >= 2^-100; a
//   tile with a smaller scale runs the same steps on x * 2^64 and s * 2^64
//   (both exact) with explicit saturation, and a zero scale gives signed
//   zero codes.
//
// Scales: s = amax / 448 as an IEEE binary32 division (the library is built
// without fast-math and keeps FP32 subnormals).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

constexpr float kE4M3Max = 448.0f;
constexpr float kFastScaleMin = 0x1p-100f;   // smallest scale of the fast path
constexpr float kMarginLo = 1.0f - 0x1p-20f;
constexpr float kMarginHi = 1.0f + 0x1p-20f;

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E4M3 value of a code (hardware decode; exact).
__device__ __forceinline__ float e4m3_dec(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(code), 0);
}

// Pack four floats into four E4M3 codes (byte i = value i), hardware RNE.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return static_cast<uint32_t>(r);
}

// Per-tile constants of the encoder.
struct TileScale {
  float s;    // stored scale fl32(amax / 448)
  float rlo;  // lower bracket multiplier (fast path)
  float rhi;  // upper bracket multiplier (fast path)
  bool fast;  // s >= 2^-100
};

__device__ __forceinline__ TileScale make_tile_scale(float amax) {
  TileScale t;
  t.s = amax / kE4M3Max;
  t.fast = t.s >= kFastScaleMin;
  const float r = __builtin_amdgcn_rcpf(t.fast ? t.s : 1.0f);
  t.rlo = r * kMarginLo;
  t.rhi = r * kMarginHi;
  return t;
}

// Decide between two adjacent codes (bracketing magnitudes) for value x and
// scale s with s >= 2^-100 (or both prescaled by 2^64).
__device__ __forceinline__ uint32_t resolve_pair(float x, float s, uint32_t c_lo, uint32_t c_hi) {
  const uint32_t m1 = c_lo & 0x7fu, m2 = c_hi & 0x7fu;
  const uint32_t small = m1 < m2 ? m1 : m2;
  const uint32_t big = m1 < m2 ? m2 : m1;
  const float mid = 0.5f * (e4m3_dec(small) + e4m3_dec(big));  // exact
  const float t = __builtin_fmaf(-mid, s, __builtin_fabsf(x));  // sign exact
  uint32_t mag;
  if (t > 0.0f) mag = big;
  else if (t < 0.0f) mag = small;
  else mag = (small & 1u) ? big : small;
  return mag | (__float_as_uint(x) >> 31 << 7);
}

// Exact code of one value, any scale (slow path).
__device__ __noinline__ uint32_t encode_general(float x, float s) {
  if (s == 0.0f) return (__float_as_uint(x) >> 31) << 7;
  float xs = x, ss = s;
  if (!(s >= kFastScaleMin)) {
    xs = x * 0x1p64f;
    ss = s * 0x1p64f;
  }
  const float r = __builtin_amdgcn_rcpf(ss);
  const float ylo = __builtin_fminf(__builtin_fmaxf(xs * (r * kMarginLo), -kE4M3Max), kE4M3Max);
  const float yhi = __builtin_fminf(__builtin_fmaxf(xs * (r * kMarginHi), -kE4M3Max), kE4M3Max);
  const uint32_t clo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(ylo, ylo, 0, false)) & 0xffu;
  const uint32_t chi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(yhi, yhi, 0, false)) & 0xffu;
  if (clo == chi) return clo;
  return resolve_pair(xs, ss, clo, chi);
}

// Encode 4 values with one tile's constants; returns the packed codes.
// Fast path when the brackets agree; per-byte repair otherwise.
__device__ __forceinline__ uint32_t encode4(const float v[4], const TileScale& t) {
  if (t.fast) {
    const uint32_t lo = cvt4(v[0] * t.rlo, v[1] * t.rlo, v[2] * t.rlo, v[3] * t.rlo);
    const uint32_t hi = cvt4(v[0] * t.rhi, v[1] * t.rhi, v[2] * t.rhi, v[3] * t.rhi);
    if (__builtin_expect(lo == hi, 1)) return lo;
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t cl = (lo >> (8 * i)) & 0xffu, ch = (hi >> (8 * i)) & 0xffu;
      const uint32_t c = (cl == ch) ? cl : resolve_pair(v[i], t.s, cl, ch);
      out |= c << (8 * i);
    }
    return out;
  }
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) out |= encode_general(v[i], t.s) << (8 * i);
  return out;
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15) of non-negative
// floats; every lane of the row gets the result.
__device__ __forceinline__ float row16_max(float v) {
  int x = __float_as_int(v);
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false));  // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xf, 0xf, false));  // row_mirror
  return __int_as_float(x);
}

// Max over all 64 lanes of non-negative floats (result in every lane).
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  int x = __float_as_int(v);
  x = max(x, __shfl_xor(x, 16));
  x = max(x, __shfl_xor(x, 32));
  return __int_as_float(x);
}

// Two floats to two bf16 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 (IEEE rounding of the default mode; FP32 subnormals
// kept).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// Debug builds with FP8BS_POISON_LDS fill a kernel's LDS with 0xFF bytes
// (NaN as FP32, and the NaN code as E4M3) before its first use, so that a
// read of LDS that the kernel never wrote changes its results.  Called at
// the top of a kernel by every thread; a no-op in the library build.
template <int BYTES>
__device__ __forceinline__ void poison_lds(void* lds) {
#ifdef FP8BS_POISON_LDS
  uint32_t* p = static_cast<uint32_t*>(lds);
  for (int i = static_cast<int>(threadIdx.x); i < BYTES / 4; i += static_cast<int>(blockDim.x))
    p[i] = 0xffffffffu;
  __syncthreads();
#else
  (void)lds;
#endif
}

// Direct global -> LDS copies through buffer descriptors.
// buffer_load_dword{,x4} ... offen lds writes lane l's 4 (16) bytes at
// M0 + 4 l (16 l).  The descriptor covers only the valid rows of the tile:
// a lane whose offset (VGPR offset + SGPR offset) is past the end reads
// zeros instead of memory, so ragged tiles need no per-lane clamping.  M0 is
// saved and restored around the copy so no compiler-owned use of M0 is
// disturbed.  The compiler does not see these as memory operations:
// completion is waited for explicitly with vmcnt before the barrier that
// publishes a stage.
typedef __attribute__((ext_vector_type(4))) int i32x4;

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = static_cast<int>(static_cast<uint32_t>(b));
  r[1] = static_cast<int>(static_cast<uint32_t>(b >> 32) & 0xffffu);  // stride 0: raw buffer
  r[2] = static_cast<int>(bytes);                                      // bytes in range
  r[3] = 0x00020000;                                                   // 32-bit data format
  return r;
}
__device__ __forceinline__ void copy16_to_lds(const i32x4& rsrc, uint32_t voff, uint32_t soff,
                                              uint32_t lds_addr) {
  uint32_t saved;
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // uniform by contract
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void copy4_to_lds(const i32x4& rsrc, uint32_t voff, uint32_t soff,
                                             uint32_t lds_addr) {
  uint32_t saved;
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // uniform by contract
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int WAIT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace fp8bs
