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
// One 256-thread workgroup per tile of 128 tokens; the tile goes through LDS
// once, so every input and output byte crosses HBM once.
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

// Tile: 128 tokens x CW channels (CW = 128 for FP8 codes, 64 for bf16, so
// a token row of the tile is 128 bytes either way).  Phase 1 copies the
// tile into LDS with coalesced 16-byte loads.  Phase 2 gives each thread 16
// consecutive tokens of CPT channels (4 bytes of each token row): the
// max-abs over a channel's 128 tokens is a reduction over the 8 lanes that
// share the channel (DPP), each thread derives the scales of only its own
// CPT channels, and each channel's 16 codes leave as one 16-byte store.
// Dwords of a row are XOR-swizzled by 8 * ((row / 16) % 4) so that the
// column reads of phase 2 see at most 2-way bank conflicts.
template <bool SRC_BF16>
__global__ __launch_bounds__(256) void requant_kernel(const uint8_t* __restrict__ in,
                                                      const float* __restrict__ s_in, int64_t T,
                                                      int64_t ld_in_bytes, int64_t lds_in,
                                                      uint8_t* __restrict__ q_out, int64_t ld_out,
                                                      float* __restrict__ s_out, int64_t lds_out) {
  constexpr int ELEM = SRC_BF16 ? 2 : 1;
  constexpr int CW = SRC_BF16 ? 64 : 128;   // channels per tile
  constexpr int CPT = SRC_BF16 ? 2 : 4;     // channels per thread
  __shared__ __align__(16) uint8_t tile[128 * 128];
  __shared__ float srow[128];

  const int tid = threadIdx.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * CW;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 128;

  // phase 1: coalesced global -> LDS, 8 chunks of 16 bytes per token row
  {
    const int ch = tid & 7;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (tid >> 3) + 32 * p;
      const int64_t t = t0 + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t < T) v = load16_nt(in + t * ld_in_bytes + c0 * ELEM + ch * 16);
      const int phys = ch ^ (2 * ((r >> 4) & 3));
      *reinterpret_cast<uint4*>(tile + r * 128 + phys * 16) = v;
    }
    if (!SRC_BF16 && tid < 128) {
      const int64_t t = t0 + tid;
      srow[tid] = (t < T) ? s_in[t * lds_in + c0 / 128] : 0.0f;
    }
  }
  __syncthreads();

  // phase 2
  const int tg = tid & 7;   // tokens 16 tg .. 16 tg + 15
  const int cg = tid >> 3;  // dword cg of every row: channels CPT cg .. CPT cg + CPT - 1
  const int dw = cg ^ (8 * (tg & 3));
  float v[CPT][16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int r = 16 * tg + t;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + r * 128 + dw * 4);
    if (SRC_BF16) {
      v[0][t] = bf16_lo(w);
      v[1 % CPT][t] = bf16_hi(w);
    } else {
      const float s1 = srow[r];
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
      v[0][t] = lo[0] * s1;  // one FP32 multiply: fl32(dec(q) * s1)
      v[1 % CPT][t] = lo[1] * s1;
      v[2 % CPT][t] = hi[0] * s1;
      v[3 % CPT][t] = hi[1] * s1;
    }
  }

  const int64_t tok = t0 + 16 * tg;
  const bool full = tok + 15 < T;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    float am = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) am = __builtin_fmaxf(am, __builtin_fabsf(v[c][t]));
    int x = __float_as_int(am);
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));   // lane ^ 1
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));   // lane ^ 2
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false));  // half-row mirror
    const TileScale ts = make_tile_scale(__int_as_float(x));
    uint32_t codes[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) codes[k] = encode4(&v[c][4 * k], ts);
    const int64_t ch = c0 + CPT * cg + c;
    uint8_t* dst = q_out + ch * ld_out + tok;
    if (full) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    } else {
      for (int k = 0; k < 16; ++k)
        if (tok + k < T) dst[k] = static_cast<uint8_t>(codes[k / 4] >> (8 * (k % 4)));
    }
    if (tg == 0) s_out[ch * lds_out + blockIdx.y] = ts.s;
  }
}

}  // namespace

hipError_t launch_requant_T_128x1(bool src_bf16, const void* in, const float* s_in, int64_t T,
                                  int64_t C, int64_t ld_in, int64_t lds_in, uint8_t* q_out,
                                  int64_t ld_out, float* s_out, int64_t lds_out, hipStream_t st) {
  const int64_t CB = src_bf16 ? C / 64 : C / 128;
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
