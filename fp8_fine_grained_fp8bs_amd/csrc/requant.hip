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
// The tile goes through LDS once, so every input and output byte crosses
// HBM once.  The same tile machinery transposes 128x128-block-quantized
// weights for the backward pass for the input (transpose_w_kernel).
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

// Tile: 128 tokens x CW channels (CW = 128 for FP8 codes, 64 for bf16, so
// a token row of the tile is 128 bytes either way).  Workgroups are
// persistent: each walks the tiles blockIdx.x, + gridDim.x, ...  The FP8
// source keeps two LDS buffers: the load unit copies the next tile (and its
// 128 input scales) global -> LDS directly while the current tile is
// re-quantized.  The bf16 and E5M6 sources keep one (16 KiB), which lets six
// workgroups share a compute unit instead of four: their loads overlap
// across workgroups instead of inside one (measured 3-8% faster cold; the
// FP8 source would spill at six waves per SIMD).
// Copies are bounded by buffer descriptors, so token rows past T read as
// zeros.  16-byte chunks of a token row are XOR-swizzled by
// 2 * ((row / 16) % 4), so that the column reads below see at most 2-way
// bank conflicts; the copy realises the swizzle by fetching, for LDS slot
// (row, p), the global chunk p ^ swizzle(row).
//
// Re-quantization: each thread takes 16 consecutive tokens of CPT channels
// (4 bytes of each token row); the max-abs over a channel's 128 tokens is a
// reduction over the 8 lanes that share the channel (DPP), each thread
// derives the scales of only its own CPT channels, and each channel's 16
// codes leave as one 16-byte store.
// FP8 source: four 256-thread workgroups per compute unit (the launch's
// grid assumes them): 4 waves per SIMD, so at most 128 VGPRs per wave.
// (Left to itself it took 130, which let only three workgroups in.)  Other
// sources: six, at most 80 VGPRs.
// Sources: kSrcFp8 (codes and 1x128 scales), kSrcBf16, kSrcE5m6 (12-bit
// E5M6 as fp8bs_encode_e5m6 packs it).  An E5M6 tile (128 tokens x 64
// channels, 96 bytes per token row) is loaded into registers (non-temporal,
// 12 bytes = 8 values per load), then decoded to bf16 by way of FP16 (an
// E5M6 code is the upper 12 bits of the FP16 encoding of its value; about 3
// instructions per value against 16 for decoding the fields with branches,
// which made this kernel bound by instruction issue) and written into the
// bf16 tile layout (swizzle included); from there on it is the bf16 path.
// Decoding is exact for finite values, so the result is that of the bf16
// source on the decoded rows, without their HBM round trip.
constexpr int kSrcFp8 = 0, kSrcBf16 = 1, kSrcE5m6 = 2;
constexpr int kXcds = 8;   // MI355X: workgroup b runs on XCD b % 8

template <int SRC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SRC == kSrcFp8 ? 4 : 6)))
void requant_kernel(const uint8_t* __restrict__ in,
                                                      const float* __restrict__ s_in, int64_t T,
                                                      int64_t ld_in_bytes, int64_t lds_in,
                                                      uint8_t* __restrict__ q_out, int64_t ld_out,
                                                      float* __restrict__ s_out, int64_t lds_out,
                                                      int64_t tiles, int64_t ctiles) {
  constexpr bool SRC_BF16 = SRC != kSrcFp8;  // the tile in LDS holds bf16 values
  constexpr int ELEM = SRC_BF16 ? 2 : 1;
  constexpr int CW = SRC_BF16 ? 64 : 128;   // channels per tile
  constexpr int CPT = SRC_BF16 ? 2 : 4;     // channels per thread
  constexpr int NB = SRC_BF16 ? 1 : 2;      // LDS tile buffers
  __shared__ __align__(16) uint8_t tile[NB][128 * 128];
  __shared__ float srow[NB][128];
  poison_lds<sizeof(tile)>(tile);
  poison_lds<sizeof(srow)>(srow);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // copy plan: copy j (0..3) of wave w moves token rows 32 j + 8 w .. + 7;
  // lane l fills LDS chunk l % 8 of row 32 j + 8 w + l / 8 with global chunk
  // (l % 8) ^ swizzle(row)
  const int crow = 8 * wave + (lane >> 3);
  const uint32_t ld_in32 = static_cast<uint32_t>(ld_in_bytes);
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * j + crow;
    voff[j] = static_cast<uint32_t>(r) * ld_in32 + static_cast<uint32_t>((lane & 7) ^ (2 * ((r >> 4) & 3))) * 16u;
  }
  const uint32_t lds_tile = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&tile[0][0]));
  const uint32_t lds_srow = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&srow[0][0]));

  auto issue = [&](int64_t t, int buf) {
    const int64_t tt = t / ctiles, cb = t - tt * ctiles;
    const int64_t t0 = tt * 128, c0 = cb * CW;
    const int64_t rows = T - t0 < 128 ? T - t0 : 128;
    const i32x4 rs = make_rsrc(in + t0 * ld_in_bytes + c0 * ELEM, static_cast<uint32_t>(rows * ld_in_bytes));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      copy16_to_lds_nt(rs, voff[j], 0u, lds_tile + buf * 16384 + (4 * j + wave) * 1024);
    if (!SRC_BF16 && wave < 2) {
      const i32x4 rss = make_rsrc(s_in + t0 * lds_in + c0 / 128, static_cast<uint32_t>(rows * lds_in * 4));
      copy4_to_lds(rss, static_cast<uint32_t>(64 * wave + lane) * static_cast<uint32_t>(lds_in * 4), 0u,
                   lds_srow + buf * 512 + wave * 256);
    }
  };

  // E5M6 load plan: item j (0..3) of thread tid is token row (tid + 256 j) / 8
  // of the tile and its 8-channel chunk (tid + 256 j) % 8; E5Regs holds the
  // 12 words of the four items
  struct E5Regs {
    u32x4 a, b, c;
  };
  auto e5_load = [&](int64_t t, E5Regs& e) {
    const int64_t tt = t / ctiles, cb = t - tt * ctiles;
    const int64_t t0 = tt * 128, c0 = cb * CW;
    const int rows = static_cast<int>(T - t0 < 128 ? T - t0 : 128);
    const uint8_t* base = in + t0 * ld_in_bytes + c0 * 3 / 2;
    uint32_t w[12];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int item = tid + 256 * j, r = item >> 3, c = item & 7;
      // rows past T are zeros, as the copies of the other sources read them
      const uint32_t* src = reinterpret_cast<const uint32_t*>(base + (r < rows ? r : 0) * ld_in_bytes + 12 * c);
      const uint32_t m = r < rows ? 0xffffffffu : 0u;
      w[3 * j] = __builtin_nontemporal_load(src) & m;
      w[3 * j + 1] = __builtin_nontemporal_load(src + 1) & m;
      w[3 * j + 2] = __builtin_nontemporal_load(src + 2) & m;
    }
    e.a = u32x4{w[0], w[1], w[2], w[3]};
    e.b = u32x4{w[4], w[5], w[6], w[7]};
    e.c = u32x4{w[8], w[9], w[10], w[11]};
  };
  auto e5_store = [&](int buf, const E5Regs& e) {
    const uint32_t w[12] = {e.a[0], e.a[1], e.a[2], e.a[3], e.b[0], e.b[1], e.b[2], e.b[3],
                            e.c[0], e.c[1], e.c[2], e.c[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int item = tid + 256 * j, r = item >> 3, c = item & 7;
      const uint4 o = bf16x8_of_e5m6x8_f16(w[3 * j], w[3 * j + 1], w[3 * j + 2]);
      *reinterpret_cast<uint4*>(&tile[buf][r * 128 + ((c ^ (2 * ((r >> 4) & 3))) << 4)]) = o;
    }
  };

  const int tg = tid & 7;   // tokens 16 tg .. 16 tg + 15
  const int cg = tid >> 3;  // dword cg of every row: channels CPT cg .. CPT cg + CPT - 1
  const int dw = cg ^ (8 * (tg & 3));

  // re-quantize tile t, which is in LDS buffer buf, and store its codes and
  // scales
  auto requant_tile = [&](int64_t t, int buf) {
    const int64_t tt = t / ctiles, cb = t - tt * ctiles;
    const int64_t t0 = tt * 128, c0 = cb * CW;
    const uint8_t* tb = &tile[buf][0];
    float v[CPT][16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 16 * tg + k;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(tb + r * 128 + dw * 4);
      if (SRC_BF16) {
        v[0][k] = bf16_lo(w);
        v[1 % CPT][k] = bf16_hi(w);
      } else {
        const float s1 = srow[buf][r];
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
        v[0][k] = lo[0] * s1;  // one FP32 multiply: fl32(dec(q) * s1)
        v[1 % CPT][k] = lo[1] * s1;
        v[2 % CPT][k] = hi[0] * s1;
        v[3 % CPT][k] = hi[1] * s1;
      }
    }
    const int64_t tok = t0 + 16 * tg;
    const bool full = tok + 15 < T;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float am = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) am = __builtin_fmaxf(am, __builtin_fabsf(v[c][k]));
      int x = __float_as_int(am);
      x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));   // lane ^ 1
      x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));   // lane ^ 2
      x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false));  // half-row mirror
      const TileScale ts = make_tile_scale(__int_as_float(x));
      const Bf16Side side = bf16_side(ts.s, __int_as_float(x));
      uint32_t codes[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        codes[k] = SRC_BF16 ? encode4_bf16(&v[c][4 * k], ts, side) : encode4(&v[c][4 * k], ts);
      const int64_t ch = c0 + CPT * cg + c;
      uint8_t* dst = q_out + ch * ld_out + tok;
      if (full) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
      } else if (tok < T) {
        for (int k = 0; k < 16; ++k)
          if (tok + k < T) dst[k] = static_cast<uint8_t>(codes[k / 4] >> (8 * (k % 4)));
      }
      if (tg == 0) s_out[ch * lds_out + tt] = ts.s;
    }
  };

  const int64_t step = gridDim.x;
  int64_t t = blockIdx.x;
  if (NB == 1) {
    // one buffer: load, re-quantize, and every wave done reading before the
    // next tile's load writes the buffer
    E5Regs r;
    for (int64_t v = t; v < tiles; v += step) {
      if (SRC == kSrcE5m6) {
        // E5M6 rows of adjacent channel tiles (96 bytes each) share cache
        // lines, so each XCD takes one contiguous range of the tiles
        // (workgroup b runs on XCD b % 8): neighbours run at the same time
        // in one L2 instead of fetching the shared lines once per XCD
        const int64_t x = v % kXcds, q = tiles / kXcds, rem = tiles % kXcds;
        t = x * q + (x < rem ? x : rem) + v / kXcds;
        e5_load(t, r);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        e5_store(0, r);
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);   // this wave's decoded rows are in LDS
      } else {
        t = v;
        issue(t, 0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      block_barrier();
      requant_tile(t, 0);
      block_barrier();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    return;
  }

  if (t < tiles) issue(t, 0);
  for (int it = 0; t < tiles; ++it) {
    const int buf = it & 1;
    const int64_t tn = t + step;
    // tile t has landed in `buf`; every wave is done with the other buffer
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    block_barrier();
    if (tn < tiles) issue(tn, buf ^ 1);
    requant_tile(t, buf);
    t = tn;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// ---------------------------------------------------------------------
// Transpose of 128x128-block-quantized weights, for the backward pass for
// the input ([p3] para 4, xn--9g3bo1gtkw0l8ubf92bgle.kr post wr_id=113503,
// splits the backward pass into a part for the input and a part for the
// weights).  dX = dY W consumes W as the B
// operand of a K-contiguous GEMM, i.e. as W^T [K][N].  The max-abs of a
// 128x128 block does not depend on its orientation, so the blocks of W^T
// are the transposed blocks of W with the same scales: the codes move as
// bytes and the scale grid is transposed; nothing is re-quantized.
//
// A tile is one 128x128 block.  The copy plan and the LDS swizzle are
// those of requant_kernel (rows are the N index, 128 code bytes each);
// each thread reads 16 consecutive rows of one dword column (4 k), turns
// the 16x4 bytes around with byte permutes, and writes 16 bytes to each
// of its 4 output rows.
// ---------------------------------------------------------------------
// transpose of a 4x4 byte block: byte c of result[c'] = byte c' of w[c]
__device__ __forceinline__ void transpose4x4(const uint32_t (&w)[4], uint32_t (&t)[4]) {
  const uint32_t x0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
  const uint32_t x1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
  const uint32_t y0 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const uint32_t y1 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  t[0] = __builtin_amdgcn_perm(y0, x0, 0x05040100u);
  t[1] = __builtin_amdgcn_perm(y0, x0, 0x07060302u);
  t[2] = __builtin_amdgcn_perm(y1, x1, 0x05040100u);
  t[3] = __builtin_amdgcn_perm(y1, x1, 0x07060302u);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void transpose_w_kernel(const uint8_t* __restrict__ q, int64_t ldq,
                                                          const float* __restrict__ s, int64_t lds,
                                                          uint8_t* __restrict__ qt, int64_t ldqt,
                                                          float* __restrict__ st, int64_t ldst,
                                                          int64_t tiles, int64_t ktiles) {
  __shared__ __align__(16) uint8_t tile[2][128 * 128];
  poison_lds<sizeof(tile)>(tile);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // copy plan (as in requant_kernel): copy j of wave w moves rows
  // 32 j + 8 w .. + 7, lane l fills LDS chunk l % 8 of its row with global
  // chunk (l % 8) ^ swizzle(row)
  const int crow = 8 * wave + (lane >> 3);
  const uint32_t ldq32 = static_cast<uint32_t>(ldq);
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * j + crow;
    voff[j] = static_cast<uint32_t>(r) * ldq32 + static_cast<uint32_t>((lane & 7) ^ (2 * ((r >> 4) & 3))) * 16u;
  }
  const uint32_t lds_tile = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&tile[0][0]));
  auto issue = [&](int64_t t, int buf) {
    const int64_t nb = t / ktiles, kb = t - nb * ktiles;
    const i32x4 rs = make_rsrc(q + nb * 128 * ldq + kb * 128, 128u * ldq32);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      copy16_to_lds_nt(rs, voff[j], 0u, lds_tile + buf * 16384 + (4 * j + wave) * 1024);
  };

  const int tg = tid & 7;   // rows 16 tg .. 16 tg + 15 of the block
  const int cg = tid >> 3;  // dword cg of every row: columns 4 cg .. 4 cg + 3
  const int dw = cg ^ (8 * (tg & 3));

  int64_t t = blockIdx.x;
  if (t < tiles) issue(t, 0);
  for (int it = 0; t < tiles; ++it) {
    const int buf = it & 1;
    const int64_t tn = t + gridDim.x;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // tile t landed (and earlier stores are done)
    block_barrier();                            // every wave is done with the other buffer
    if (tn < tiles) issue(tn, buf ^ 1);

    const int64_t nb = t / ktiles, kb = t - nb * ktiles;
    const uint8_t* tb = &tile[buf][0];
    uint32_t out[4][4];  // out[c][i]: bytes of rows 16 tg + 4 i .. + 3 in column 4 cg + c
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[4], tr[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = *reinterpret_cast<const uint32_t*>(tb + (16 * tg + 4 * i + k) * 128 + dw * 4);
      transpose4x4(w, tr);
#pragma unroll
      for (int c = 0; c < 4; ++c) out[c][i] = tr[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint8_t* dst = qt + (kb * 128 + 4 * cg + c) * ldqt + nb * 128 + 16 * tg;
      *reinterpret_cast<uint4*>(dst) = make_uint4(out[c][0], out[c][1], out[c][2], out[c][3]);
    }
    if (tid == 0) st[kb * ldst + nb] = s[nb * lds + kb];
    t = tn;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

}  // namespace

hipError_t launch_requant_T_128x1(int src, const void* in, const float* s_in, int64_t T,
                                  int64_t C, int64_t ld_in, int64_t lds_in, uint8_t* q_out,
                                  int64_t ld_out, float* s_out, int64_t lds_out, hipStream_t st) {
  const int64_t CB = src == kSrcFp8 ? C / 128 : C / 64;
  const int64_t TB = (T + 127) / 128;
  const int64_t tiles = CB * TB;
  // four 33 KiB workgroups (FP8 source) or six 16 KiB ones per compute unit
  // of a 256-CU MI355X
  const int64_t cap = src == kSrcFp8 ? 1024 : 1536;
  const int64_t grid = tiles < cap ? tiles : cap;
  const uint8_t* s8 = static_cast<const uint8_t*>(in);
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  if (src == kSrcBf16)
    hipLaunchKernelGGL(requant_kernel<kSrcBf16>, g, b, 0, st, s8, s_in, T, ld_in * 2, lds_in, q_out, ld_out,
                       s_out, lds_out, tiles, CB);
  else if (src == kSrcE5m6)
    hipLaunchKernelGGL(requant_kernel<kSrcE5m6>, g, b, 0, st, s8, s_in, T, ld_in, lds_in, q_out, ld_out,
                       s_out, lds_out, tiles, CB);
  else
    hipLaunchKernelGGL(requant_kernel<kSrcFp8>, g, b, 0, st, s8, s_in, T, ld_in, lds_in, q_out, ld_out,
                       s_out, lds_out, tiles, CB);
  return hipGetLastError();
}

hipError_t launch_transpose_w_128x128(const uint8_t* q, int64_t N, int64_t K, int64_t ldq,
                                      const float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                                      float* st, int64_t ldst, hipStream_t stream) {
  const int64_t ktiles = K / 128;
  const int64_t tiles = (N / 128) * ktiles;
  // four 32 KiB workgroups per compute unit of a 256-CU MI355X
  const int64_t grid = tiles < 1024 ? tiles : 1024;
  hipLaunchKernelGGL(transpose_w_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, q,
                     ldq, s, lds, qt, ldqt, st, ldst, tiles, ktiles);
  return hipGetLastError();
}

}  // namespace fp8bs
