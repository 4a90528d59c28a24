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
//   BF16 tiles (every x and amax with at most 8 significant bits) need no
//   repair step at all (encode4_bf16).  Write v = 448 x / amax, the quotient
//   by the unrounded scale; x / s = v (amax / 448) / s differs from v by at
//   most 2^-24 relatively.  Brackets that differ put a midpoint mu within
//   2^-19.9 of x / s, hence within 2^-19.8 of v.  But 448 x - mu amax is an
//   integer combination of 7 X 2^(a+6) and N A 2^(b+c) (x = X 2^a,
//   amax = A 2^b, mu = N 2^c with X, A < 2^8, N < 2^5), so it is zero or at
//   least 2^-13 of mu amax: differing brackets mean v = mu exactly.  Then
//   x / s lies below mu when s was rounded up (448 s > amax), above it when
//   s was rounded down, and on it when s is exact (a tie: the even code);
//   the sign of 448 s - amax comes exactly from one fma per tile.  In
//   random BF16 data such brackets differ for about 0.5 % of the values
//   (amax significands with small odd factors), i.e. in most waves.
//
// Scales: s = fl32(amax / 448), the correctly rounded quotient (div448, or
// the IEEE binary32 division where that does not apply; the library is
// built without fast-math and keeps FP32 subnormals).
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
// The first conversion writes the low half of its result and keeps the
// high half of the old value it is given, which the second conversion then
// overwrites: any old value will do, and a's own bits (a register that dies
// here) spare the zeroing move a literal 0 would cost.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
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

// fl32(a / 448) in three operations: q0 = a * fl32(1/448), the exact
// remainder a - 448 q0 (one FMA), q0 corrected by remainder * fl32(1/448).
// Equal to the IEEE quotient for every binary32 a whose quotient is at
// least 2^-100 (checked on the CPU over every significand in exact integer
// arithmetic, tests/test_div448.py); smaller or non-finite quotients need
// the IEEE division.
__device__ __forceinline__ float div448(float a) {
  constexpr float kInv448 = 1.0f / 448.0f;
  const float q0 = a * kInv448;
  const float r = __builtin_fmaf(-q0, 448.0f, a);
  return __builtin_fmaf(r, kInv448, q0);
}

__device__ __forceinline__ TileScale make_tile_scale(float amax) {
  TileScale t;
  t.s = div448(amax);
  t.fast = t.s >= kFastScaleMin;
  // below 2^-100 (and for zero or a non-finite amax) the IEEE division,
  // branched around: it is eleven instructions against div448's three
  if (__builtin_expect(!t.fast, 0)) t.s = amax / kE4M3Max;
  const float r = __builtin_amdgcn_rcpf(t.fast ? t.s : 1.0f);
  t.rlo = r * kMarginLo;
  t.rhi = r * kMarginHi;
  return t;
}

// Per-tile choice for differing brackets of a BF16 tile (see the top of this
// file): the upper code where the exact quotient lies above the midpoint
// (the scale was rounded down), the even code on an exact tie (the scale is
// exact), the lower code otherwise.  As byte masks for resolve_brackets.
struct Bf16Side {
  uint32_t up;    // 0x01010101: take the upper code
  uint32_t even;  // all ones: take the even code
};
__device__ __forceinline__ Bf16Side bf16_side(float s, float amax) {
  const float d = __builtin_fmaf(s, kE4M3Max, -amax);  // 448 s - amax, sign exact
  return {d < 0.0f ? 0x01010101u : 0u, d == 0.0f ? 0xffffffffu : 0u};
}
// Packed codes of two bracketing conversions: where a byte differs the two
// codes are adjacent magnitudes (same sign, hi = lo + 1, so bit 0 differs);
// add 1 to lo there when the upper or the even (lo odd) code is chosen.  No
// carry: lo's magnitude is then at most 0x7D.
__device__ __forceinline__ uint32_t resolve_brackets(uint32_t lo, uint32_t hi, Bf16Side k) {
  return lo + ((lo ^ hi) & 0x01010101u & (k.up | (lo & k.even)));
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

// Repair of a word whose brackets differ somewhere (s >= 2^-100), without
// branches: in every byte the midpoint mu of the two codes' magnitudes
// (exact: adjacent E4M3 values sum exactly) decides by the exact sign of
// |x| - mu s = fma(-(dec(lo) + dec(hi)), s / 2, |x|); the upper code is
// taken where that is positive, or zero with an odd lower code (ties to
// even).  Bytes whose brackets agree keep lo.  The sign test reads the FP32
// bits as an integer: positive > 0, +0 = 0, negative < 0 (an exact zero
// from the fma is +0).
__device__ __forceinline__ uint32_t repair_word(const float v[4], float s, uint32_t lo, uint32_t hi) {
  const int mlo = static_cast<int>(lo & 0x7f7f7f7fu), mhi = static_cast<int>(hi & 0x7f7f7f7fu);
  const auto l01 = __builtin_amdgcn_cvt_pk_f32_fp8(mlo, false), l23 = __builtin_amdgcn_cvt_pk_f32_fp8(mlo, true);
  const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(mhi, false), h23 = __builtin_amdgcn_cvt_pk_f32_fp8(mhi, true);
  const float sum[4] = {l01[0] + h01[0], l01[1] + h01[1], l23[0] + h23[0], l23[1] + h23[1]};
  const float hs = 0.5f * s;
  uint32_t up = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = __builtin_fmaf(-sum[i], hs, __builtin_fabsf(v[i]));
    const int key = __float_as_int(t) + static_cast<int>((lo >> (8 * i)) & 1u);
    up |= (key > 0 ? 1u : 0u) << (8 * i);
  }
  return lo + ((lo ^ hi) & 0x01010101u & up);
}

// Encode 4 values with one tile's constants; returns the packed codes.
// Fast path when the brackets agree; the word's repair otherwise.
__device__ __forceinline__ uint32_t encode4(const float v[4], const TileScale& t) {
  if (t.fast) {
    const uint32_t lo = cvt4(v[0] * t.rlo, v[1] * t.rlo, v[2] * t.rlo, v[3] * t.rlo);
    const uint32_t hi = cvt4(v[0] * t.rhi, v[1] * t.rhi, v[2] * t.rhi, v[3] * t.rhi);
    if (__builtin_expect(lo == hi, 1)) return lo;
    return repair_word(v, t.s, lo, hi);
  }
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) out |= encode_general(v[i], t.s) << (8 * i);
  return out;
}

// encode4 for a BF16 tile (values and amax with at most 8 significant
// bits): differing brackets resolve by the tile's side, no repair step.
__device__ __forceinline__ uint32_t encode4_bf16(const float v[4], const TileScale& t, Bf16Side k) {
  if (__builtin_expect(t.fast, 1)) {
    const uint32_t lo = cvt4(v[0] * t.rlo, v[1] * t.rlo, v[2] * t.rlo, v[3] * t.rlo);
    const uint32_t hi = cvt4(v[0] * t.rhi, v[1] * t.rhi, v[2] * t.rhi, v[3] * t.rhi);
    return resolve_brackets(lo, hi, k);
  }
  return encode4(v, t);
}

// E5M6 (12-bit: sign, 5 exponent bits with bias 15, 6 mantissa bits) to
// bf16, exact: every E5M6 value is a bf16 value.
__device__ __forceinline__ uint32_t bf16_of_e5m6(uint32_t c) {
  const uint32_t sign = (c >> 11) << 15;
  const uint32_t e = (c >> 6) & 31u, m = c & 63u;
  uint32_t mag;
  if (e == 31u) mag = m ? 0x7FC0u : 0x7F80u;
  else if (e == 0u) mag = __float_as_uint(static_cast<float>(m) * 0x1p-20f) >> 16;  // exact
  else mag = ((e + 112u) << 7) | (m << 1);
  return sign | mag;
}

// Eight packed E5M6 values (96 bits, value i in bits 12 i .. 12 i + 11 of
// d0 | d1 << 32 | d2 << 64) to eight bf16 values, two per word.
__device__ __forceinline__ uint4 bf16x8_of_e5m6x8(uint32_t d0, uint32_t d1, uint32_t d2) {
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
  return o;
}

// The same eight values through FP16: an E5M6 code is the upper 12 bits of
// the FP16 encoding of its value (sign, 5-bit exponent with bias 15,
// subnormals, infinity and NaN alike), so code << 4 is an FP16 pattern.
// Its FP32 conversion is exact and has at most 7 significant bits, so the
// upper half of that FP32 is the bf16 value.  About 3 instructions per
// value, without branches.  Finite codes and infinities give the bit
// patterns of bf16x8_of_e5m6x8; a NaN code gives a NaN of the code's sign
// whose payload is not the canonical one (for callers whose contract
// excludes NaN inputs).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_of_e5m6x2_f16(uint32_t x) {
  // x: code 2k in bits 0..11, code 2k + 1 in bits 12..23 (bits above: any)
  // x << 4 holds code 2k << 4 in its lower half; a 16-bit shift by 4 of the
  // upper half brings code 2k + 1 (bits 16..27) to bits 20..31
  const u16x2_t z = __builtin_bit_cast(u16x2_t, x << 4) << u16x2_t{0, 4};
  const f16x2_t h = __builtin_bit_cast(f16x2_t, z);
  const float lo = static_cast<float>(h.x), hi = static_cast<float>(h.y);
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);   // upper halves
}
__device__ __forceinline__ uint4 bf16x8_of_e5m6x8_f16(uint32_t d0, uint32_t d1, uint32_t d2) {
  uint4 o;
  o.x = bf16x2_of_e5m6x2_f16(d0);
  o.y = bf16x2_of_e5m6x2_f16(__builtin_amdgcn_alignbit(d1, d0, 24));
  o.z = bf16x2_of_e5m6x2_f16(__builtin_amdgcn_alignbit(d2, d1, 16));
  o.w = bf16x2_of_e5m6x2_f16(d2 >> 8);
  return o;
}

// Two bf16 values with every NaN made the canonical quiet NaN of its sign
// (0x7FC0 / 0xFFC0).  The NaNs of bf16x2_of_e5m6x2_f16 are quiet, so their
// magnitudes lie in 0x7FC0..0x7FFF above every other value: a signed 16-bit
// min with 0x7FC0 clamps the positive ones, an unsigned min with 0xFFC0 the
// negative ones (0xFFC0..0xFFFF), and no other pattern moves.
typedef short i16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t canonical_nan_bf16x2(uint32_t w) {
  const i16x2_t a = __builtin_elementwise_min(__builtin_bit_cast(i16x2_t, w), i16x2_t{0x7FC0, 0x7FC0});
  const u16x2_t b = __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a), u16x2_t{0xFFC0, 0xFFC0});
  return __builtin_bit_cast(uint32_t, b);
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
// The same with the non-temporal hint, for data a kernel reads once: such a
// copy does not allocate in the caches, so it evicts no dirty lines of other
// data on its way (measured: requant and weight transpose 19-28% faster
// with the caches full of dirty lines, level otherwise).
__device__ __forceinline__ void copy16_to_lds_nt(const i32x4& rsrc, uint32_t voff, uint32_t soff,
                                                 uint32_t lds_addr) {
  uint32_t saved;
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // uniform by contract
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen nt lds\n\ts_mov_b32 m0, %0"
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
