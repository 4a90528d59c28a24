// gemm.hip -- block-scaled FP8 GEMM and its grouped (MoE) form for gfx950.
//
// D = A * B^T with A [M][K], B [N][K] E4M3 codes (both K-contiguous) and
// FP32 scales per 128-wide K group: sa per (row m, group g); sb per
// (128-row block of B, g) or per (row n, g).
//
// [p1] para 2 (xn--9g3bo1gtkw0l8ubf92bgle.kr post wr_id=32373): the
// per-group scales along K are multiplied in as part of dequantization on
// the general-purpose ALUs; [p1] para 3 and [p2] para 1 (why-be.why-be.co.kr
// post wr_id=73620): the matrix-unit partial sums are promoted into FP32
// accumulators; [p3] para 4 (xn--9g3bo1gtkw0l8ubf92bgle.kr post
// wr_id=113503) and [p4] para 1: the promotion is overlapped with the
// matrix unit; [p4] para 4 (bestpmk.kr post wr_id=299512): FP8 inputs, BF16
// or FP32 outputs.
//
// gfx950 mapping
// * One K group of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4 per 16x16
//   output block, issued with a zero accumulator; its FP32 result P_g is
//   promoted with one VALU FMA per output element, acc = fma(P_g, sa*sb,
//   acc).  The VALU work (4 FMAs per 32-cycle MFMA) runs beside the matrix
//   core.  (The FP8 MFMA itself keeps only ~13 bits below the largest
//   product inside each 8-product chunk, so promoting once per group is what
//   bounds the error, as on the hardware the report describes.)
// * The MFMA "A" operand is the B tile and its "B" operand the A tile, so
//   each lane ends up holding 4 consecutive output columns of one row:
//   8-byte (BF16) or 16-byte (FP32) stores in the epilogue, and one A-scale
//   per lane per 16-row block.
// * Workgroup tile 128 (M) x 256 (N), 512 threads = 2 x 4 waves of 64 x 64
//   (other shapes selectable with FP8BS_GEMM_CFG).
//   Per K group the A tile (16 KiB) and B tile (32 KiB) go global ->
//   registers -> LDS; two LDS stages and two register stages put the global
//   loads two K groups ahead of the MFMAs.  16-byte chunks are XOR-swizzled
//   with row bits 1..3 so 16 lanes reading 16 rows hit 64 distinct banks.
// * Tiles are handed out XCD-aware: the 8 XCDs each take a contiguous range
//   of the tile order, and the order walks 4 M-tiles x all N-tiles per
//   group, so the ~32 workgroups resident on one XCD share A and B panels
//   in that XCD's L2.
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

typedef __attribute__((ext_vector_type(8))) int v8i;
typedef __attribute__((ext_vector_type(4))) float v4f;

constexpr int GROUP_M = 4;     // M-tiles per group of the tile order
constexpr int NUM_XCD = 8;

// Workgroup tile BM x BN, WM x WN waves of (BM/WM) x (BN/WN).
template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = 64 * WM * WN;         // threads
  static constexpr int MB = BM / WM / 16;         // 16-row blocks per wave
  static constexpr int NB = BN / WN / 16;         // 16-column blocks per wave
  static constexpr int CA = BM * 8 / NT;          // A chunks per thread per K group
  static constexpr int CB = BN * 8 / NT;          // B chunks per thread per K group
  static constexpr int RSTEP = NT / 8;            // rows between a thread's chunks
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert(CA >= 1 && CB >= 1 && BM * 8 % NT == 0 && BN * 8 % NT == 0, "staging");
  static_assert(NT >= BM + BN, "one scale slot per thread");
};

#ifndef FP8BS_GEMM_CFG
#define FP8BS_GEMM_CFG 2
#endif
#if FP8BS_GEMM_CFG == 0
using MainCfg = Cfg<256, 128, 4, 2>;
#elif FP8BS_GEMM_CFG == 1
using MainCfg = Cfg<128, 128, 2, 2>;
#elif FP8BS_GEMM_CFG == 2
using MainCfg = Cfg<128, 256, 2, 4>;
#else
using MainCfg = Cfg<256, 256, 4, 4>;
#endif

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* d;
  const int32_t* offsets;  // grouped only
  int64_t lda, ldsa, ldb, ldsb, ldd;
  int64_t M, N, K;
  int32_t E;               // grouped only
  int32_t tiles_m;         // (upper bound of) M tiles
  int32_t tiles_n;
};

__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // cbsz = blgp = 0: E4M3 operands; literal zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Byte offset of logical 16-byte chunk `ch` of tile row `r` in LDS.
__device__ __forceinline__ int swz(int r, int ch) { return r * 128 + ((ch ^ ((r >> 1) & 7)) << 4); }

// Workgroup id -> tile, XCD-aware (see the header comment).
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& vm, int& nt) {
  const int total = tiles_m * tiles_n;
  const int q = total / NUM_XCD, r = total % NUM_XCD;
  const int x = bid % NUM_XCD, local = bid / NUM_XCD;
  const int t = x * q + (x < r ? x : r) + local;
  const int group = GROUP_M * tiles_n;
  const int first_m = (t / group) * GROUP_M;
  const int gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int rr = t % group;
  vm = first_m + rr % gm;
  nt = rr / gm;
}

// Per-thread staging registers of one K group.
template <class C>
struct Stage {
  u32x4 a[C::CA];
  u32x4 b[C::CB];
  float s;
};

template <class C>
__device__ __forceinline__ void fetch(Stage<C>& st, const uint8_t* const (&ga)[C::CA],
                                      const uint8_t* const (&gb)[C::CB], const float* gs, int64_t g) {
#pragma unroll
  for (int i = 0; i < C::CA; ++i) st.a[i] = *reinterpret_cast<const u32x4*>(ga[i] + g * 128);
#pragma unroll
  for (int i = 0; i < C::CB; ++i) st.b[i] = *reinterpret_cast<const u32x4*>(gb[i] + g * 128);
  st.s = gs[g];
}

// Registers -> one LDS stage.  Every thread stores its scale: slots
// 0..BM-1 are the A scales of the tile rows, BM.. the B scales (one per
// tile row in row mode, one per 128-wide column block in block mode), the
// rest are never read.
template <class C>
__device__ __forceinline__ void stash(const Stage<C>& st, uint8_t* la, uint8_t* lb, float* ls,
                                      int tid, int ld_r, int ld_ch) {
#pragma unroll
  for (int i = 0; i < C::CA; ++i) *reinterpret_cast<u32x4*>(la + swz(ld_r + C::RSTEP * i, ld_ch)) = st.a[i];
#pragma unroll
  for (int i = 0; i < C::CB; ++i) *reinterpret_cast<u32x4*>(lb + swz(ld_r + C::RSTEP * i, ld_ch)) = st.b[i];
  ls[tid] = st.s;
}

// One K group on one LDS stage: MB x NB MFMAs and their promotions per wave.
template <class C, bool BROW>
__device__ __forceinline__ void compute(v4f (&acc)[C::MB][C::NB], const uint8_t* la, const uint8_t* lb,
                                        const float* ls, float sbv, int wm, int wn, int lane) {
  constexpr int TM = C::MB * 16, TN = C::NB * 16;
  const float* lsa = ls;
  const float* lsb = ls + C::BM;
  // block mode: this wave's B block scale (staged in slot BM + block)
  if (!BROW) sbv = lsb[(wn * TN) / 128];
  const int fr = lane & 15;
  const int kc = lane >> 4;  // k chunks kc and kc + 4 (any permutation shared by A and B is valid)
  v8i fb[C::NB];
#pragma unroll
  for (int j = 0; j < C::NB; ++j) {
    const int r = wn * TN + j * 16 + fr;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(lb + swz(r, kc));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(lb + swz(r, kc + 4));
    fb[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  float sbn[C::NB][4];
  if (BROW) {
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(lsb + wn * TN + j * 16 + 4 * kc);
      sbn[j][0] = v.x; sbn[j][1] = v.y; sbn[j][2] = v.z; sbn[j][3] = v.w;
    }
  }
  v8i fa[C::MB];
  float sam[C::MB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
    const int r = wm * TM + i * 16 + fr;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(la + swz(r, kc));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(la + swz(r, kc + 4));
    fa[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    sam[i] = lsa[r];
  }
  // Keep the matrix core fed: raise this wave's issue priority for the MFMA
  // block and ask the scheduler to interleave the LDS reads with the MFMAs.
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_iglp_opt(0);
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
    const float sc = sam[i] * sbv;
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const v4f part = mfma_16x16x128_fp8(fb[j], fa[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s = BROW ? sam[i] * sbn[j][q] : sc;
        acc[i][j][q] = __builtin_fmaf(part[q], s, acc[i][j][q]);
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

template <class C, bool OUT_F32, bool BROW, bool GROUPED>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmArgs p) {
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __align__(16) uint8_t lds_a[2][BM * 128];
  __shared__ __align__(16) uint8_t lds_b[2][BN * 128];
  __shared__ __align__(16) float lds_s[2][C::NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t G = p.K / 128;

  // ---- tile ------------------------------------------------------------
  int vm, nt;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, vm, nt);
  const int64_t n0 = static_cast<int64_t>(nt) * BN;
  int64_t m0, m_end;
  const uint8_t* bmat = p.b;
  const float* sbmat = p.sb;
  if (GROUPED) {
    int64_t mt = vm;
    int e = 0;
    m0 = -1;
    m_end = 0;
    for (; e < p.E; ++e) {
      const int64_t r0 = p.offsets[e], r1 = p.offsets[e + 1];
      const int64_t cnt = r1 - r0;
      const int64_t tiles = cnt > 0 ? (cnt + BM - 1) / BM : 0;
      if (mt < tiles) {
        m0 = r0 + mt * BM;
        m_end = r1 < p.M ? r1 : p.M;
        break;
      }
      mt -= tiles;
    }
    if (e == p.E || m0 < 0 || m0 >= m_end) return;  // uniform per workgroup
    bmat = p.b + static_cast<int64_t>(e) * p.N * p.K;
    sbmat = p.sb + static_cast<int64_t>(e) * ((p.N + 127) / 128) * G;
  } else {
    m0 = static_cast<int64_t>(vm) * BM;
    m_end = p.M;
  }

  // ---- staging layout: thread t moves 16-byte chunk (t & 7) of rows
  //      (t >> 3) + RSTEP i of the A tile (i < CA) and of the B tile (i < CB)
  const int ld_ch = tid & 7;
  const int ld_r = tid >> 3;
  const uint8_t* ga[C::CA];
  const uint8_t* gb[C::CB];
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    int64_t r = m0 + ld_r + C::RSTEP * i;
    r = r < m_end ? r : m_end - 1;
    ga[i] = p.a + r * p.lda + ld_ch * 16;
  }
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    int64_t r = n0 + ld_r + C::RSTEP * i;
    r = r < p.N ? r : p.N - 1;
    gb[i] = bmat + r * p.ldb + ld_ch * 16;
  }
  // scales: threads t < BM fetch sa of row m0 + t; threads BM .. BM+BN-1
  // fetch sb of row n0 + t - BM in row mode; every other thread re-reads row m0's
  // sa (a valid address, value unused) so the loop has no branch
  const float* gs;
  if (tid < BM) {
    int64_t r = m0 + tid;
    r = r < m_end ? r : m_end - 1;
    gs = p.sa + r * p.ldsa;
  } else if (BROW && tid < BM + BN) {
    int64_t r = n0 + tid - BM;
    r = r < p.N ? r : p.N - 1;
    gs = sbmat + r * p.ldsb;
  } else if (!BROW && tid < BM + BN / 128) {
    // block mode: the B block scales of this tile's 128-wide column blocks
    int64_t blk = n0 / 128 + (tid - BM);
    const int64_t last_blk = (p.N - 1) / 128;
    blk = blk < last_blk ? blk : last_blk;
    gs = sbmat + blk * p.ldsb;
  } else {
    gs = p.sa + m0 * p.ldsa;
  }
  // block mode: a wave's columns lie inside one 128-wide block of B
  static_assert(BROW || (128 % (C::NB * 16) == 0), "wave columns must not straddle a B block");

  v4f acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  Stage<C> s0, s1;
  fetch(s0, ga, gb, gs, 0);
  fetch(s1, ga, gb, gs, G > 1 ? 1 : 0);
  stash(s0, lds_a[0], lds_b[0], lds_s[0], tid, ld_r, ld_ch);
  __syncthreads();

  // Pair of iterations (g, g + 1): set s0 is refilled with group g + 2 while
  // stage 0 (group g) is multiplied, then set s1 (group g + 1) goes to stage
  // 1; symmetrically for g + 1.  The loop body has no branch: prefetch
  // indices past the end are clamped to the last group (re-read, never
  // multiplied), so the compiler can keep two groups of loads in flight and
  // interleave the promotion FMAs with the MFMAs.
  const int64_t last = G - 1;
  int64_t g = 0;
  for (; g + 2 <= G; g += 2) {
    fetch(s0, ga, gb, gs, g + 2 < last ? g + 2 : last);
    compute<C, BROW>(acc, lds_a[0], lds_b[0], lds_s[0], 0.0f, wm, wn, lane);
    stash(s1, lds_a[1], lds_b[1], lds_s[1], tid, ld_r, ld_ch);
    __syncthreads();
    fetch(s1, ga, gb, gs, g + 3 < last ? g + 3 : last);
    compute<C, BROW>(acc, lds_a[1], lds_b[1], lds_s[1], 0.0f, wm, wn, lane);
    stash(s0, lds_a[0], lds_b[0], lds_s[0], tid, ld_r, ld_ch);
    __syncthreads();
  }
  if (g < G)  // odd G: stage 0 holds the last group
    compute<C, BROW>(acc, lds_a[0], lds_b[0], lds_s[0], 0.0f, wm, wn, lane);

  // ---- epilogue: lane holds columns n .. n+3 of row m per 16x16 block ----
  const int fr = lane & 15;
  const int kc = lane >> 4;
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
    const int64_t m = m0 + wm * (C::MB * 16) + i * 16 + fr;
    if (m >= m_end) continue;
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const int64_t n = n0 + wn * (C::NB * 16) + j * 16 + 4 * kc;
      if (n >= p.N) continue;
      const v4f v = acc[i][j];
      if (OUT_F32) {
        float* dst = static_cast<float*>(p.d) + m * p.ldd + n;
        if (n + 3 < p.N) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int q = 0; q < 4 && n + q < p.N; ++q) dst[q] = v[q];
        }
      } else {
        uint16_t* dst = static_cast<uint16_t*>(p.d) + m * p.ldd + n;
        const uint32_t b0 = f32_to_bf16_rne(v[0]), b1 = f32_to_bf16_rne(v[1]);
        const uint32_t b2 = f32_to_bf16_rne(v[2]), b3 = f32_to_bf16_rne(v[3]);
        if (n + 3 < p.N) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
          const uint32_t bb[4] = {b0, b1, b2, b3};
          for (int q = 0; q < 4 && n + q < p.N; ++q) dst[q] = static_cast<uint16_t>(bb[q]);
        }
      }
    }
  }
}

template <class C, bool GROUPED>
hipError_t dispatch(const GemmArgs& args, bool brow, bool out_f32, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(args.tiles_m) * args.tiles_n;
  const dim3 grid(static_cast<unsigned>(total)), block(C::NT);
  if (out_f32) {
    if (brow) hipLaunchKernelGGL((gemm_kernel<C, true, true, GROUPED>), grid, block, 0, st, args);
    else hipLaunchKernelGGL((gemm_kernel<C, true, false, GROUPED>), grid, block, 0, st, args);
  } else {
    if (brow) hipLaunchKernelGGL((gemm_kernel<C, false, true, GROUPED>), grid, block, 0, st, args);
    else hipLaunchKernelGGL((gemm_kernel<C, false, false, GROUPED>), grid, block, 0, st, args);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const float* sa, int64_t lda, int64_t ldsa,
                       const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                       bool bscale_row, void* d, int64_t ldd, bool out_f32,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  GemmArgs args{};
  args.a = a; args.sa = sa; args.b = b; args.sb = sb; args.d = d; args.offsets = nullptr;
  args.lda = lda; args.ldsa = ldsa; args.ldb = ldb; args.ldsb = ldsb; args.ldd = ldd;
  args.M = M; args.N = N; args.K = K; args.E = 0;
  using C = MainCfg;
  const int64_t tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
  args.tiles_m = static_cast<int32_t>(tm);
  args.tiles_n = static_cast<int32_t>(tn);
  return dispatch<C, false>(args, bscale_row, out_f32, st);
}

hipError_t launch_grouped_gemm(const uint8_t* a, const float* sa, int64_t ldsa,
                               const uint8_t* b, const float* sb, const int32_t* offsets,
                               int32_t E, int64_t M_total, void* d, bool out_f32,
                               int64_t N, int64_t K, hipStream_t st) {
  GemmArgs args{};
  args.a = a; args.sa = sa; args.b = b; args.sb = sb; args.d = d; args.offsets = offsets;
  args.lda = K; args.ldsa = ldsa; args.ldb = K; args.ldsb = K / 128; args.ldd = N;
  args.M = M_total; args.N = N; args.K = K; args.E = E;
  // upper bound of the per-expert M-tile count: each expert adds at most one
  // partial tile
  using C = MainCfg;
  const int64_t tm = (M_total + C::BM - 1) / C::BM + E, tn = (N + C::BN - 1) / C::BN;
  if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
  args.tiles_m = static_cast<int32_t>(tm);
  args.tiles_n = static_cast<int32_t>(tn);
  return dispatch<C, true>(args, false, out_f32, st);
}

}  // namespace fp8bs
