// gemm_bf16a.hip -- block-scaled FP8 GEMM whose A operand arrives in BF16 and
// is quantized in 1x128 tiles inside the GEMM (gfx950).
//
// [p2] para 1 (why-be.why-be.co.kr post wr_id=73620): separate quantization
// reads 128 BF16 activations from HBM, writes the FP8 values back to HBM
// and reads them again for the MMA.  Here the BF16 rows of A go straight
// from HBM into LDS, each 1x128 tile (one row of one K group) is quantized
// there exactly as fp8bs_quant_act_1x128 quantizes it ([p1] para 3:
// online max-abs per 1x128 tile, s = fl32(amax / 448), nearest-even E4M3 of
// x / s, saturated), and the codes feed the MFMAs from LDS: the FP8
// activation never crosses HBM.  Optionally the workgroups of the first
// column of tiles also store the codes and scales, the FP8 cache of the
// activation for the backward pass ([p1] para 4).
//
// The GEMM arithmetic is that of fp8bs_gemm with 128x128 B scales: one
// v_mfma_f32_16x16x128_f8f6f4 per 16x16 block and K group with the same
// fragment layout, its FP32 partial promoted by acc = fma(P, sa * sb, acc)
// in K-group order, so D is bit for bit the D of fp8bs_gemm on these codes.
//
// Each tile of A is quantized once per tile of B it meets, so the form
// pays where N is small (a few 256-column tiles): the HBM traffic of A is
// its BF16 bytes once instead of BF16 + 2 x FP8.
//
// Tile 64 (M) x 256 (N), 512 threads = 2 x 4 waves of 32 x 64.  LDS holds
// 4 raw stages of A (64 BF16 rows of one K group, 16 KiB each) and 3 code
// stages of B (256 rows of 128 E4M3 codes, 32 KiB each): 160 KiB.
// Iteration g copies B of g + 2 and the raw A of g + 3, quantizes A of
// g + 1 in place and multiplies g, so every copy has two iterations to
// land.  A tile of A is quantized inside its own raw stage: a row's 128
// codes take 8 of the row's 16 byte chunks (those of the row's parity,
// XOR-swizzled so that 16 lanes reading 16 rows hit distinct banks) and its
// scale one of the other 8.  The B block scales (one per 128 columns and K
// group) are read with scalar loads one group ahead.
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

typedef __attribute__((ext_vector_type(8))) int v8i;
typedef __attribute__((ext_vector_type(4))) float v4f;

constexpr int BM = 64, BN = 256, NT = 512;
constexpr int WM = 2, WN = 4;            // wave grid
constexpr int MB = BM / WM / 16;         // 16-row blocks per wave (2)
constexpr int NB = BN / WN / 16;         // 16-column blocks per wave (4)
constexpr int RAW = BM * 256;            // BF16 A of one K group: 16 KiB
constexpr int NRAW = 4;
constexpr int BST = BN * 128;            // E4M3 B of one K group: 32 KiB
constexpr int NBST = 3;
constexpr int RAW_OFF = 0;
constexpr int B_OFF = NRAW * RAW;
constexpr int LDS_BYTES = B_OFF + NBST * BST;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// B stage: byte offset of logical 16-byte chunk `ch` of code row `r` (row
// bits 1..3 XOR-swizzle the chunks, so 16 lanes reading 16 rows hit
// distinct banks).
__device__ __forceinline__ int swz(int r, int ch) { return r * 128 + ((ch ^ ((r >> 1) & 7)) << 4); }
// Raw stage after quantization (256-byte rows): chunk `ch` of row r's codes
// at chunk position (2 ch + r % 2) ^ (2 ((r >> 1) & 7)), its scale at the
// start of position 2 ((r >> 1) & 7) + 1 - r % 2 (the other parity).
__device__ __forceinline__ int cpos(int r, int ch) {
  return r * 256 + (((2 * ch + (r & 1)) ^ (((r >> 1) & 7) << 1)) << 4);
}
__device__ __forceinline__ int spos(int r) { return r * 256 + ((2 * ((r >> 1) & 7) + ((r & 1) ^ 1)) << 4); }

__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // cbsz = blgp = 0: E4M3 operands; literal zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Max over the 16 lanes of a DPP row of non-negative floats (as integers);
// the row moves feed the max directly.
__device__ __forceinline__ int row16_imax(int x) {
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, true));    // quad_perm [1,0,3,2]
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, true));    // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, true));   // row_half_mirror
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, true));   // row_mirror
  return x;
}

constexpr int kOutBf16 = 0, kOutF32 = 1;

struct Bf16aArgs {
  const uint16_t* x;
  uint8_t* qx;   // optional code output (nullptr: not stored)
  float* sx;
  const uint8_t* b;
  const float* sb;
  void* d;
  int64_t ldx, ldqx, ldsx, ldb, ldsb, ldd;
  int64_t M, N, K;
  int32_t tiles_m, tiles_n;
};

template <int OUT>
__global__ __launch_bounds__(NT) void gemm_bf16a_kernel(Bf16aArgs p) {
  __shared__ __align__(16) uint8_t lds[LDS_BYTES];
  poison_lds<LDS_BYTES>(lds);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int G = static_cast<int>(p.K / 128);

  // XCD-aware tile order: the workgroups of one XCD (blockIdx % 8) take the
  // column tiles of the same row tile together, so that they share the
  // BF16 rows of A in that XCD's L2.
  const int x = blockIdx.x % 8, j = blockIdx.x / 8;
  const int mt = (j / p.tiles_n) * 8 + x, nt = j % p.tiles_n;
  if (mt >= p.tiles_m) return;  // uniform per workgroup
  const int64_t m0 = static_cast<int64_t>(mt) * BM, n0 = static_cast<int64_t>(nt) * BN;
  const int64_t rows_a = p.M - m0 < BM ? p.M - m0 : BM;
  const int64_t rows_b = p.N - n0 < BN ? p.N - n0 : BN;
  const bool store_codes = p.qx != nullptr && nt == 0;

  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds[0]));
  const uint32_t ldx_b = static_cast<uint32_t>(p.ldx * 2);
  const uint32_t ldb = static_cast<uint32_t>(p.ldb);
  // descriptors bound every copy to the tile's valid rows (rows past the
  // end read as zeros); row offsets are in the VGPR offset, the SGPR offset
  // carries only the K group's column offset
  const i32x4 rs_x = make_rsrc(p.x + m0 * p.ldx, static_cast<uint32_t>(rows_a) * ldx_b);
  const i32x4 rs_b = make_rsrc(p.b + n0 * p.ldb, static_cast<uint32_t>(rows_b) * ldb);
  // this wave's B block scales: block (n0 + 64 wn) / 128 of B, if it has rows
  // (read through the constant address space: wave-uniform loads of memory
  // the kernel never writes become scalar loads, outside the vector
  // memory counter that paces the copies)
  typedef __attribute__((address_space(4))) const float cfloat;
  const int64_t sbblk = (n0 + wn * NB * 16) / 128;
  const cfloat* const sbrow = (const cfloat*)((n0 + wn * NB * 16 < p.N) ? p.sb + sbblk * p.ldsb : p.sb);

  // raw A copy k (0, 1) of this wave: rows 4 (wave + 8k) .. + 3, lane l
  // fetches 16 bytes of row l / 16 (lane-linear in LDS: row r at r * 256)
  uint32_t xoff[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    xoff[k] = static_cast<uint32_t>(4 * (wave + 8 * k) + (lane >> 4)) * ldx_b + (lane & 15) * 16;
  // B copy k (0..3): rows 8 (wave + 8k) .. + 7, lane l fetches row l / 8,
  // global chunk (l & 7) ^ swizzle(row), into LDS slot l
  uint32_t boff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 8 * (wave + 8 * k) + (lane >> 3);
    boff[k] = static_cast<uint32_t>(r) * ldb + (((lane & 7) ^ ((r >> 1) & 7)) * 16);
  }

  // past the last group the copies are clamped to it: they refill a free
  // stage with valid data and keep the per-iteration copy count fixed
  auto issue_b = [&](int t, int st) {
    const int tc = t < G - 1 ? t : G - 1;
    const uint32_t gk = static_cast<uint32_t>(tc) * 128u;
    const uint32_t base = lds_base + B_OFF + st * BST;
#pragma unroll
    for (int k = 0; k < 4; ++k) copy16_to_lds(rs_b, boff[k], gk, base + (wave + 8 * k) * 1024);
  };
  auto issue_x = [&](int t, int st) {
    const int tc = t < G - 1 ? t : G - 1;
    const uint32_t gk = static_cast<uint32_t>(tc) * 256u;
    const uint32_t base = lds_base + RAW_OFF + st * RAW;
#pragma unroll
    for (int k = 0; k < 2; ++k) copy16_to_lds(rs_x, xoff[k], gk, base + (wave + 8 * k) * 1024);
  };

  // quantization of one K group in raw stage st, in place: wave w takes
  // rows 8w .. 8w + 7, a 16-lane DPP row one 1x128 tile (row), 8 bf16 per
  // lane; lane `sub` of the row holds elements 8 sub .. 8 sub + 7 of rows
  // 8w + dr and 8w + 4 + dr, both tiles in one straight-line pass (scales
  // >= 2^-100: two bracketing conversions, differing ones resolved by the
  // tile's side, as the standalone quantizer's BF16 path does); tiles with
  // smaller or non-finite scales go through that quantizer's general code.  A row's raw bytes are
  // all read (the row maximum needs them) before its codes are written over
  // them, and no other wave touches the row.  The codes and scales stay in
  // registers for the optional store to HBM.
  const int sub = lane & 15, dr = lane >> 4;
  uint2 kcode[2];
  float kscale[2];
  auto quantize = [&](int st) {
    uint8_t* raw = lds + RAW_OFF + st * RAW;
    const int r0 = 8 * wave + dr, r1 = r0 + 4;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(raw + r0 * 256 + sub * 16);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(raw + r1 * 256 + sub * 16);
    const float f0[8] = {bf16_lo(w0[0]), bf16_hi(w0[0]), bf16_lo(w0[1]), bf16_hi(w0[1]),
                         bf16_lo(w0[2]), bf16_hi(w0[2]), bf16_lo(w0[3]), bf16_hi(w0[3])};
    const float f1[8] = {bf16_lo(w1[0]), bf16_hi(w1[0]), bf16_lo(w1[1]), bf16_hi(w1[1]),
                         bf16_lo(w1[2]), bf16_hi(w1[2]), bf16_lo(w1[3]), bf16_hi(w1[3])};
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a0 = __builtin_fmaxf(a0, __builtin_fabsf(f0[i]));
      a1 = __builtin_fmaxf(a1, __builtin_fabsf(f1[i]));
    }
    a0 = __int_as_float(row16_imax(__float_as_int(a0)));
    a1 = __int_as_float(row16_imax(__float_as_int(a1)));
    float s0 = div448(a0), s1 = div448(a1);
    const bool fast = s0 >= kFastScaleMin && s1 >= kFastScaleMin;   // false for NaN
    const float q0 = __builtin_amdgcn_rcpf(s0), q1 = __builtin_amdgcn_rcpf(s1);
    const float lo0 = q0 * kMarginLo, hi0 = q0 * kMarginHi;
    const float lo1 = q1 * kMarginLo, hi1 = q1 * kMarginHi;
    uint32_t c[4], h[4];
    c[0] = cvt4(f0[0] * lo0, f0[1] * lo0, f0[2] * lo0, f0[3] * lo0);
    h[0] = cvt4(f0[0] * hi0, f0[1] * hi0, f0[2] * hi0, f0[3] * hi0);
    c[1] = cvt4(f0[4] * lo0, f0[5] * lo0, f0[6] * lo0, f0[7] * lo0);
    h[1] = cvt4(f0[4] * hi0, f0[5] * hi0, f0[6] * hi0, f0[7] * hi0);
    c[2] = cvt4(f1[0] * lo1, f1[1] * lo1, f1[2] * lo1, f1[3] * lo1);
    h[2] = cvt4(f1[0] * hi1, f1[1] * hi1, f1[2] * hi1, f1[3] * hi1);
    c[3] = cvt4(f1[4] * lo1, f1[5] * lo1, f1[6] * lo1, f1[7] * lo1);
    h[3] = cvt4(f1[4] * hi1, f1[5] * hi1, f1[6] * hi1, f1[7] * hi1);
    // differing brackets resolve by each tile's side (exact for BF16 tiles)
    const Bf16Side k0 = bf16_side(s0, a0), k1 = bf16_side(s1, a1);
    c[0] = resolve_brackets(c[0], h[0], k0);
    c[1] = resolve_brackets(c[1], h[1], k0);
    c[2] = resolve_brackets(c[2], h[2], k1);
    c[3] = resolve_brackets(c[3], h[3], k1);
    if (__builtin_expect(!fast, 0)) {
      const TileScale t0 = make_tile_scale(a0), t1 = make_tile_scale(a1);
      s0 = t0.s;
      s1 = t1.s;
      c[0] = encode4(f0, t0);
      c[1] = encode4(f0 + 4, t0);
      c[2] = encode4(f1, t1);
      c[3] = encode4(f1 + 4, t1);
    }
    kcode[0] = make_uint2(c[0], c[1]);
    kcode[1] = make_uint2(c[2], c[3]);
    kscale[0] = s0;
    kscale[1] = s1;
    *reinterpret_cast<uint2*>(raw + cpos(r0, sub >> 1) + (sub & 1) * 8) = kcode[0];
    *reinterpret_cast<uint2*>(raw + cpos(r1, sub >> 1) + (sub & 1) * 8) = kcode[1];
    if (sub == 0) {
      *reinterpret_cast<float*>(raw + spos(r0)) = s0;
      *reinterpret_cast<float*>(raw + spos(r1)) = s1;
    }
  };
  auto store_quantized = [&](int t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * wave + 4 * h + dr;
      if (m0 + r < p.M) {
        *reinterpret_cast<uint2*>(p.qx + (m0 + r) * p.ldqx + static_cast<int64_t>(t) * 128 + sub * 8) = kcode[h];
        if (sub == 0) p.sx[(m0 + r) * p.ldsx + t] = kscale[h];
      }
    }
  };

  // fragments of one K group for this wave (the layout of fp8bs_gemm: lane
  // (fr, kc) reads row fr of a 16-row block, chunks kc and kc + 4)
  const int fr = lane & 15, kc = lane >> 4;
  v4f acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int jn = 0; jn < NB; ++jn) acc[i][jn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- prologue: raw A of groups 0, 1, 2 and B of groups 0, 1 in flight;
  //      quantize group 0.  Six copies per wave per iteration afterwards.
  issue_x(0, 0);
  issue_b(0, 0);
  issue_x(1, 1);
  issue_b(1, 1);
  issue_x(2, 2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(12));  // raw A 0 (copies complete in order)
  block_barrier();
  quantize(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(6));   // raw A 1 and B 0 as well
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
  block_barrier();
  if (store_codes) store_quantized(0);
  float sbv = sbrow[0];

  int bst = 0;   // B stage of group g (g % 3)
  for (int g = 0; g < G; ++g) {
    const int bst2 = bst == 0 ? 2 : bst - 1;   // (g + 2) % 3
    // copies: B of g + 2 into the stage read in iteration g - 1, raw A of
    // g + 3 into the raw stage of g - 1 (both free since the last barrier)
    issue_b(g + 2, bst2);
    issue_x(g + 3, (g + 3) & 3);
    const float sbv_next = sbrow[__builtin_amdgcn_readfirstlane(g + 1 < G ? g + 1 : G - 1)];
    // quantize g + 1 (its raw A landed before the last barrier)
    if (g + 1 < G) quantize((g + 1) & 3);
    // multiply g
    const uint8_t* la = lds + RAW_OFF + (g & 3) * RAW;
    const uint8_t* lb = lds + B_OFF + bst * BST;
    v8i fb[NB], fa[MB];
#pragma unroll
    for (int jn = 0; jn < NB; ++jn) {
      const int r = (wn * NB + jn) * 16 + fr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(lb + swz(r, kc));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(lb + swz(r, kc + 4));
      fb[jn] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    float sam[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = (wm * MB + i) * 16 + fr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(la + cpos(r, kc));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(la + cpos(r, kc + 4));
      fa[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      sam[i] = *reinterpret_cast<const float*>(la + spos(r));
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const float sc = sam[i] * sbv;
#pragma unroll
      for (int jn = 0; jn < NB; ++jn) {
        const v4f part = mfma_16x16x128_fp8(fb[jn], fa[i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][jn][q] = __builtin_fmaf(part[q], sc, acc[i][jn][q]);
      }
    }
    // B of g + 1 and raw A of g + 2 (and everything before them) complete;
    // this iteration's six copies may remain in flight.  This wave's LDS
    // reads and writes are done.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(6));
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    block_barrier();
    if (store_codes && g + 1 < G) store_quantized(g + 1);
    sbv = sbv_next;
    bst = bst == 2 ? 0 : bst + 1;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the clamped copies past the last group
  block_barrier();

  // ---- epilogue through the B stages (padded rows): lane (fr, kc) holds
  //      columns 4 kc .. 4 kc + 3 of row fr of each 16x16 block
  constexpr int OB = OUT == kOutBf16 ? 2 : 4;
  constexpr int ROWB = BN * OB + 16;
  constexpr int CPR = BN * OB / 16;
  static_assert(BM * ROWB <= NBST * BST, "output staging");
  uint8_t* const ob = lds + B_OFF;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = (wm * MB + i) * 16 + fr;
#pragma unroll
    for (int jn = 0; jn < NB; ++jn) {
      const int c = (wn * NB + jn) * 16 + 4 * kc;
      const v4f vv = acc[i][jn];
      uint8_t* dst = ob + r * ROWB + c * OB;
      if (OUT == kOutF32) *reinterpret_cast<float4*>(dst) = make_float4(vv[0], vv[1], vv[2], vv[3]);
      else *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2_rne(vv[0], vv[1]), pack_bf16x2_rne(vv[2], vv[3]));
    }
  }
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
  block_barrier();
  uint8_t* dbase = static_cast<uint8_t*>(p.d);
  const int64_t ldd_b = p.ldd * OB;
  for (int ch = tid; ch < BM * CPR; ch += NT) {
    const int r = ch / CPR, cc = ch % CPR;
    const int64_t m = m0 + r;
    const int c0 = cc * (16 / OB);
    if (m >= p.M || c0 >= rows_b) continue;
    const uint8_t* src = ob + r * ROWB + cc * 16;
    uint8_t* dst = dbase + m * ldd_b + (n0 + c0) * OB;
    if (c0 + 16 / OB <= rows_b) {
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst));
    } else {
      for (int e = 0; e < (rows_b - c0) * OB; ++e) dst[e] = src[e];
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16a(const uint16_t* x, int64_t ldx, uint8_t* qx, int64_t ldqx, float* sx,
                             int64_t ldsx, const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                             void* d, int64_t ldd, bool out_f32, int64_t M, int64_t N, int64_t K,
                             hipStream_t st) {
  Bf16aArgs a{};
  a.x = x; a.qx = qx; a.sx = sx; a.b = b; a.sb = sb; a.d = d;
  a.ldx = ldx; a.ldqx = ldqx; a.ldsx = ldsx; a.ldb = ldb; a.ldsb = ldsb; a.ldd = ldd;
  a.M = M; a.N = N; a.K = K;
  const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int64_t blocks = (tm + 7) / 8 * 8 * tn;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  a.tiles_m = static_cast<int32_t>(tm);
  a.tiles_n = static_cast<int32_t>(tn);
  if (out_f32) hipLaunchKernelGGL(gemm_bf16a_kernel<kOutF32>, dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, st, a);
  else hipLaunchKernelGGL(gemm_bf16a_kernel<kOutBf16>, dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace fp8bs
