// requant.hip -- backward re-quantization of 1x128 tiles into 128x1 tiles.
//
// [p1] para 3 (xn--9g3bo1gtkw0l8ubf92bgle.kr post wr_id=32373): in the
// backward pass the activation tiles are converted from 1x128 to 128x1;
// [p1] para 4: the activations were cached in FP8 for the backward pass of
// the Linear operator.  Each value is dequantized with one FP32 multiply,
// v = fl32(dec(q) * s1), every run of 128 consecutive tokens of a channel is
// re-quantized as one tile, and the result is written channel-major so the
// token dimension becomes the contiguous K of the weight-gradient GEMM.
//
// One 256-thread workgroup per 128-token x 128-channel tile; the tile goes
// through LDS once (an XOR swizzle of 16-byte chunks keeps both the
// row-wise writes and the 4-token-by-16-channel reads free of bank
// conflicts), so every input and output byte crosses HBM once.
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

template <bool SRC_BF16>
__global__ __launch_bounds__(256) void requant_kernel(const uint8_t* __restrict__ in,
                                                      const float* __restrict__ s_in, int64_t T,
                                                      int64_t ld_in_bytes, int64_t lds_in,
                                                      uint8_t* __restrict__ q_out, int64_t ld_out,
                                                      float* __restrict__ s_out, int64_t lds_out) {
  constexpr int ELEM = SRC_BF16 ? 2 : 1;
  constexpr int ROWB = 128 * ELEM;   // bytes per token row of the tile
  constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;     // rows per pass of the workgroup
  __shared__ __align__(16) uint8_t tile[128 * ROWB];
  __shared__ float srow[128];

  const int tid = threadIdx.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 128;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 128;

  // phase 1: coalesced global -> LDS
  {
    const int ch = tid % CPR;
#pragma unroll
    for (int p = 0; p < 128 / RPP; ++p) {
      const int r = tid / CPR + RPP * p;
      const int64_t t = t0 + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t < T)
        v = load16_nt(in + t * ld_in_bytes + c0 * ELEM + ch * 16);
      const int phys = ch ^ ((r >> 2) & 7);
      *reinterpret_cast<uint4*>(tile + r * ROWB + phys * 16) = v;
    }
    if (!SRC_BF16 && tid < 128) {
      const int64_t t = t0 + tid;
      srow[tid] = (t < T) ? s_in[t * lds_in + c0 / 128] : 0.0f;
    }
  }
  __syncthreads();

  // phase 2: 4 tokens x 16 channels per thread
  const int lane = tid & 63;
  const int tr = lane & 31;                       // tokens 4tr .. 4tr+3
  const int tc = (tid >> 6) * 2 + (lane >> 5);    // channels 16tc .. 16tc+15
  float v[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * tr + i;
    const int f = (r >> 2) & 7;
    if (SRC_BF16) {
      const uint4 a = *reinterpret_cast<const uint4*>(tile + r * ROWB + (((2 * tc) ^ f) * 16));
      const uint4 b = *reinterpret_cast<const uint4*>(tile + r * ROWB + (((2 * tc + 1) ^ f) * 16));
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[i][2 * k] = bf16_lo(w[k]);
        v[i][2 * k + 1] = bf16_hi(w[k]);
      }
    } else {
      const uint4 a = *reinterpret_cast<const uint4*>(tile + r * ROWB + ((tc ^ f) * 16));
      const float s1 = srow[r];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[k]), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[k]), true);
        v[i][4 * k + 0] = lo[0] * s1;
        v[i][4 * k + 1] = lo[1] * s1;
        v[i][4 * k + 2] = hi[0] * s1;
        v[i][4 * k + 3] = hi[1] * s1;
      }
    }
  }

  const int64_t tok = t0 + 4 * tr;
  const bool full = tok + 3 < T;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float am = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0][j]), __builtin_fabsf(v[1][j])),
                               __builtin_fmaxf(__builtin_fabsf(v[2][j]), __builtin_fabsf(v[3][j])));
    am = row16_max(am);
    am = __int_as_float(max(__float_as_int(am), __shfl_xor(__float_as_int(am), 16)));
    const TileScale ts = make_tile_scale(am);
    const float col[4] = {v[0][j], v[1][j], v[2][j], v[3][j]};
    const uint32_t codes = encode4(col, ts);
    const int64_t c = c0 + 16 * tc + j;
    uint8_t* dst = q_out + c * ld_out + tok;
    if (full) {
      *reinterpret_cast<uint32_t*>(dst) = codes;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (tok + k < T) dst[k] = static_cast<uint8_t>(codes >> (8 * k));
    }
    if (tr == 0) s_out[c * lds_out + blockIdx.y] = ts.s;
  }
}

}  // namespace

hipError_t launch_requant_T_128x1(bool src_bf16, const void* in, const float* s_in, int64_t T,
                                  int64_t C, int64_t ld_in, int64_t lds_in, uint8_t* q_out,
                                  int64_t ld_out, float* s_out, int64_t lds_out, hipStream_t st) {
  const int64_t CB = C / 128;
  const int64_t TB = (T + 127) / 128;
  if (CB > 0x7fffffff || TB > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(CB), static_cast<unsigned>(TB));
  const uint8_t* src = static_cast<const uint8_t*>(in);
  if (src_bf16)
    hipLaunchKernelGGL(requant_kernel<true>, grid, dim3(256), 0, st, src, s_in, T, ld_in * 2,
                       lds_in, q_out, ld_out, s_out, lds_out);
  else
    hipLaunchKernelGGL(requant_kernel<false>, grid, dim3(256), 0, st, src, s_in, T, ld_in,
                       lds_in, q_out, ld_out, s_out, lds_out);
  return hipGetLastError();
}

}  // namespace fp8bs
