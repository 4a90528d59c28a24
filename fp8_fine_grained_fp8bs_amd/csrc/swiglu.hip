// swiglu.hip -- SwiGLU of the cached gate and up halves, quantized in 1x128
// tiles for the down-projection (gfx950).
//
// [p1] para 4 (xn--9g3bo1gtkw0l8ubf92bgle.kr post wr_id=32373) and [p4]
// para 3 (bestpmk.kr post wr_id=299512) cache the inputs of the SwiGLU
// operator and recompute its output in the backward pass; [p1] para 3
// quantizes a GEMM's input in 1x128 tiles along its K; [p2] para 1
// (why-be.why-be.co.kr post wr_id=73620) counts the HBM round trip of a
// separate quantization.  This kernel reads the two cached BF16 halves once
// and writes the down-projection's E4M3 codes and 1x128 scales of
// h = silu(g) u directly (5 bytes per element instead of 4 + 2 for a BF16
// h and 2 + 1 for quantizing it), and optionally h itself in BF16 (the
// backward pass's recompute, which re-quantizes it along tokens).
//
// h is computed in FP32: sigma(g) from e = exp(-|g|) (never overflows):
// 1 / (1 + e) for g >= 0, e / (1 + e) for g < 0; h = (g sigma) u, within a
// few units in the last place of the exact value.
// The codes and scales are those of the FP32 tile quantizer (s = fl32(amax
// / 448) by IEEE division, the exact two-bracket encoding) applied to these
// FP32 values.  A 16-lane DPP row takes one tile, 8 values per lane; each
// row keeps two tiles of loads in flight (measured faster than one, four or
// eight tiles: fewer registers, more resident waves).
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

constexpr int kTilesPerRow = 2;   // tiles of one DPP row, loaded before any is encoded

// e^-a for a >= 0 by the hardware's 2^x (v_exp_f32, within about one unit
// in the last place) after the argument reduction of Cody and Waite
// (Software Manual for the Elementary Functions, 1980): log2(e) is split
// into a binary32 head and tail, y = -a * head is rounded, and the exact
// residual of that product plus -a * tail (r, |r| <= 2^-17) enters to first
// order: 2^(y + r) = 2^y (1 + r ln 2), the dropped term below 2^-35.
__device__ __forceinline__ float exp_neg(float a) {
  constexpr float kLog2eHi = 0x1.715476p+0f;   // fl32(log2 e)
  constexpr float kLog2eLo = 0x1.4ae0cp-26f;   // fl32(log2 e - kLog2eHi)
  constexpr float kLn2 = 0x1.62e43p-1f;        // fl32(ln 2)
  const float y = -a * kLog2eHi;
  float r = __builtin_fmaf(-a, kLog2eHi, -y);
  r = __builtin_fmaf(-a, kLog2eLo, r);
  const float p = __builtin_amdgcn_exp2f(y);
  return __builtin_fmaf(p, r * kLn2, p);
}

__device__ __forceinline__ float swiglu1(float g, float u) {
  const float e = exp_neg(__builtin_fabsf(g));
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  const float sig = g >= 0.0f ? r : e * r;
  return (g * sig) * u;
}

template <bool CODES, bool HOUT>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const uint16_t* __restrict__ g, int64_t ldg,
                                                           const uint16_t* __restrict__ u, int64_t ldu,
                                                           int64_t T, int G, uint8_t* __restrict__ q,
                                                           int64_t ldq, float* __restrict__ s, int64_t lds,
                                                           uint16_t* __restrict__ h, int64_t ldh) {
  const int tid = threadIdx.x;
  const int sub = tid & 15;
  const int64_t rid = static_cast<int64_t>(blockIdx.x) * 16 + (tid >> 4);   // DPP row of the grid
  const int64_t tiles = T * G;
  // the row's consecutive tiles: (token, group) of the first, then stepped
  const int64_t tile0 = rid * kTilesPerRow;
  int64_t tk[kTilesPerRow];
  int ck[kTilesPerRow];
  {
    int64_t t = tile0 / G;
    int c = static_cast<int>(tile0 - t * G);
#pragma unroll
    for (int k = 0; k < kTilesPerRow; ++k) {
      tk[k] = t;
      ck[k] = c;
      if (++c == G) {
        c = 0;
        ++t;
      }
    }
  }
  u32x4 vg[kTilesPerRow], vu[kTilesPerRow];
#pragma unroll
  for (int k = 0; k < kTilesPerRow; ++k) {
    const int64_t tile = tile0 + k;
    if (tile < tiles) {
      const int64_t t = tk[k];
      const int c = ck[k];
      const uint4 a = load16_nt(g + t * ldg + c * 128 + sub * 8);
      const uint4 b = load16_nt(u + t * ldu + c * 128 + sub * 8);
      vg[k] = u32x4{a.x, a.y, a.z, a.w};
      vu[k] = u32x4{b.x, b.y, b.z, b.w};
    } else {
      vg[k] = u32x4{0u, 0u, 0u, 0u};
      vu[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int k = 0; k < kTilesPerRow; ++k) {
    const int64_t tile = tile0 + k;
    float hv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hv[2 * j] = swiglu1(bf16_lo(vg[k][j]), bf16_lo(vu[k][j]));
      hv[2 * j + 1] = swiglu1(bf16_hi(vg[k][j]), bf16_hi(vu[k][j]));
    }
    uint2 cw = make_uint2(0u, 0u);
    float sc = 0.0f;
    if (CODES) {
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(hv[i]));
      am = row16_max(am);   // every lane of the DPP row runs this (uniform per row)
      const TileScale ts = make_tile_scale(am);
      sc = ts.s;
      cw = make_uint2(encode4(hv, ts), encode4(hv + 4, ts));
    }
    if (tile < tiles) {
      const int64_t t = tk[k];
      const int c = ck[k];
      if (CODES) {
        *reinterpret_cast<uint2*>(q + t * ldq + c * 128 + sub * 8) = cw;
        if (sub == 0) s[t * lds + c] = sc;
      }
      if (HOUT) {
        const u32x4 hb = {pack_bf16x2_rne(hv[0], hv[1]), pack_bf16x2_rne(hv[2], hv[3]),
                          pack_bf16x2_rne(hv[4], hv[5]), pack_bf16x2_rne(hv[6], hv[7])};
        __builtin_nontemporal_store(hb, reinterpret_cast<u32x4*>(h + t * ldh + c * 128 + sub * 8));
      }
    }
  }
}

}  // namespace

hipError_t launch_swiglu_quant_1x128(const uint16_t* g, int64_t ldg, const uint16_t* u, int64_t ldu,
                                     int64_t T, int64_t I, uint8_t* q, int64_t ldq, float* s,
                                     int64_t lds, uint16_t* h, int64_t ldh, hipStream_t st) {
  const int G = static_cast<int>(I / 128);
  const int64_t rows = (T * G + kTilesPerRow - 1) / kTilesPerRow;   // DPP rows
  const int64_t blocks = (rows + 15) / 16;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (q != nullptr && h != nullptr)
    hipLaunchKernelGGL((swiglu_quant_kernel<true, true>), grid, block, 0, st, g, ldg, u, ldu, T, G, q, ldq, s, lds, h, ldh);
  else if (q != nullptr)
    hipLaunchKernelGGL((swiglu_quant_kernel<true, false>), grid, block, 0, st, g, ldg, u, ldu, T, G, q, ldq, s, lds, h, ldh);
  else
    hipLaunchKernelGGL((swiglu_quant_kernel<false, true>), grid, block, 0, st, g, ldg, u, ldu, T, G, q, ldq, s, lds, h, ldh);
  return hipGetLastError();
}

}  // namespace fp8bs
