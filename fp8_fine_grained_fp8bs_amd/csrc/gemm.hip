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
//   each lane ends up holding 4 consecutive output columns of one row and
//   needs one A-scale per 16-row block.
// * Workgroup tile 128 (M) x 256 (N), 512 threads = 2 x 4 waves of 64 x 64
//   (row-mode B scales: 128 x 128, 2 x 4 waves of 64 x 32).
//   The A tile (16 KiB) and B tile (32 KiB) of a K group are copied
//   global -> LDS by the load unit itself (buffer_load_dwordx4 ... lds: no
//   staging registers, no LDS write instructions), into three LDS stages:
//   while group g is multiplied from registers, the fragments of group g+1
//   are read from LDS and groups g+2 and g+3 are in flight.  16-byte chunks
//   are XOR-swizzled with row bits 1..3 so 16 lanes reading 16 rows hit 64
//   distinct banks; the direct loads write that layout by fetching, for LDS
//   slot (row, chunk p), the global chunk p ^ swizzle(row).  Buffer
//   descriptors bound each copy to the tile's valid rows (rows past the
//   end read as zeros): every row offset is in the VGPR offset, which the
//   range check covers; the SGPR offset carries only the K group's column
//   offset, which keeps a valid row's address inside that row.
// * The FP32 scales travel in blocks of 4 K groups through a 3-slot LDS
//   ring, one quarter block per K group: each lane fetches 4 consecutive
//   groups of one row, so a row's scales cost one cache line per 4 groups
//   instead of one per group.
// * Tiles are handed out XCD-aware: the 8 XCDs each take a contiguous range
//   of the tile order, and the order walks 8 M-tiles x all N-tiles per
//   group, so the ~32 workgroups resident on one XCD (8 M-tiles x 4 N-tiles
//   at a time: the B panel of a 128x256 tile is twice the A panel) share A
//   and B panels in that XCD's L2.
// * Workgroups are persistent (one per compute unit).  The finished tile
//   goes out through LDS with 16-byte stores, as BF16, FP32, or E4M3 codes
//   with one scale per 1x128 tile along N (the next layer's activation
//   quantization fused into the epilogue).  With K a multiple of 512 the
//   workgroup's next tile is copied during the current tile's last K groups
//   (the tile stream, below); otherwise its first groups are copied after
//   the last one.
#include <hip/hip_runtime.h>

#include "fp8bs_device.h"
#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

typedef __attribute__((ext_vector_type(8))) int v8i;
typedef __attribute__((ext_vector_type(4))) float v4f;

constexpr int GROUP_M = 8;          // M-tiles per group of the tile order
constexpr int GROUP_M_EXPERTS = 4;  // the same for the grouped form (see tile_of)
constexpr int NUM_XCD = 8;
constexpr int SBLK = 4;        // K groups per scale block
constexpr int NSLOT = 3;       // scale blocks resident in LDS

// Workgroup tile BM x BN, WM x WN waves of (BM/WM) x (BN/WN), three LDS
// stages: the fragments of the next K group are read from LDS while the
// current one is multiplied (two fragment register sets).
template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NSTAGE = 3;
  static constexpr int NW = WM * WN;              // waves
  static constexpr int NT = 64 * NW;              // threads
  static constexpr int MB = BM / WM / 16;         // 16-row blocks per wave
  static constexpr int NB = BN / WN / 16;         // 16-column blocks per wave
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int DPW = (BM + BN) / 8 / NW;  // 1 KiB tile copies per wave per K group
  // Scale ring: NSLOT slots, each with the scales of SBLK consecutive K
  // groups; A scales as [BM/16][SBLK][16] floats, B scales as
  // [BN/16][SBLK][16] (row mode) or [SBLK][16] (block mode) floats.
  static constexpr int SAW = BM / 64;             // waves copying A scales
  static constexpr int SA_BYTES = BM * SBLK * 4;
  static constexpr int sbw(bool brow) { return brow ? BN / 64 : 1; }
  static constexpr int sb_bytes(bool brow) { return brow ? BN * SBLK * 4 : 256; }
  static constexpr int slot_bytes(bool brow) { return SA_BYTES + sb_bytes(brow); }
  static constexpr int sc_area() { return NSTAGE * STAGE; }
  static constexpr int dummy_off(bool brow) { return sc_area() + NSLOT * slot_bytes(brow); }
  // the next tile's four buffer descriptors (A, B, A scales, B scales)
  static constexpr int next_off(bool brow) { return dummy_off(brow) + 256; }
  static constexpr int lds_bytes(bool brow) { return next_off(brow) + 64; }
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert((BM + BN) % (8 * NW) == 0, "tile copies must split evenly over the waves");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale copies move 16-row units, SBLK per lane row");
};

using MainCfg = Cfg<128, 256, 2, 4>;
// Row-scale mode holds 16 more scales per fragment set: narrower wave tiles.
using RowCfg = Cfg<128, 128, 2, 4>;
// Block mode on problems too small to fill the chip with 128x256 tiles:
// when every 128x128 tile fits in one round of the persistent grid, the
// half-size tiles keep more compute units busy.  A round of 128x128 tiles
// takes about 0.63 of a round of 128x256 tiles (measured), so they lose as
// soon as they need more rounds than the large tiles: 4096 x 576 x 7168
// 49.8 against 65.8 us and 2048 x 2048 x 7168 50.6 against 65.4 us, but
// 4096 x 1536 x 7168 90.2 against 71.2 us.  Every output element takes the
// same MFMAs and promotions either way, so the results are identical.
using SmallCfg = Cfg<128, 128, 2, 4>;
constexpr int64_t kGridCap = 256;   // persistent workgroups: one per compute unit

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* d;                 // output (E4M3 codes when the output is quantized)
  float* s_out;            // 1x128 scales of a quantized output
  const int32_t* offsets;  // grouped only
  int64_t lda, ldsa, ldb, ldsb, ldd, lds_out;
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

// Tile t of the group order: groups of GM M-tiles by all tile columns, the
// M-tiles of a group adjacent in t, so that the tiles that run at one time
// share A rows and B columns.
template <int GM>
__device__ __forceinline__ void tile_in_groups(int t, int tiles_m, int tiles_n, int& vm, int& nt) {
  const int group = GM * tiles_n;
  const int first_m = (t / group) * GM;
  const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int rr = t % group;
  vm = first_m + rr % gm;
  nt = rr / gm;
}

// Workgroup id -> tile, XCD-aware (see the header comment): each XCD takes
// one contiguous range of the group order.
template <int GM>
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& vm, int& nt) {
  const int total = tiles_m * tiles_n;
  const int q = total / NUM_XCD, r = total % NUM_XCD;
  const int x = bid % NUM_XCD, local = bid / NUM_XCD;
  tile_in_groups<GM>(x * q + (x < r ? x : r) + local, tiles_m, tiles_n, vm, nt);
}

// The grouped form's order.  Tiles of different experts cost differently:
// a small expert's B panels serve few M-tiles, so its tiles fetch more B per
// tile.  With contiguous XCD ranges the last XCD holds the smallest experts
// of a skewed routing and finishes last.  So the XCDs take chunks of the
// group order round-robin instead: one chunk is one round of an XCD's
// workgroups (kChunk consecutive tiles, which share A rows and B columns in
// that XCD's L2), and every XCD gets chunks from every part of the order.
// Measured on 8 experts (16384 tokens): Zipf counts 3-5% faster at
// K = 2048, equal at K = 7168; equal counts 8% (K = 2048) and 12% (K =
// 7168) faster.  Dense shapes, whose tiles cost alike, keep tile_of.
// Virtual ids past the last chunk round's tiles map to no tile (false).
constexpr int kChunk = 32;   // workgroups of one XCD in a 256-workgroup launch
__device__ __forceinline__ bool tile_of_chunked(int bid, int tiles_m, int tiles_n, int& vm, int& nt) {
  const int x = bid % NUM_XCD, local = bid / NUM_XCD;
  const int t = ((local / kChunk) * NUM_XCD + x) * kChunk + local % kChunk;
  if (t >= tiles_m * tiles_n) return false;
  tile_in_groups<GROUP_M_EXPERTS>(t, tiles_m, tiles_n, vm, nt);
  return true;
}

// Copies for the GEMM loop: M0 is set without being saved or restored.  The
// compiler never uses M0 in this file's kernels (tests/test_gemm_m0.py checks
// the generated code), so nothing it relies on is disturbed.
__device__ __forceinline__ void gemm_copy16(const i32x4& rsrc, uint32_t voff, uint32_t soff,
                                            uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // uniform by contract
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void gemm_copy4(const i32x4& rsrc, uint32_t voff, uint32_t soff,
                                           uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // uniform by contract
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// This lane's index in its wave, computed by the asm statement itself where
// it stands (it can be neither hoisted nor kept across the code around it).
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Fragments (and their scales) of one K group for one wave.
template <class C>
struct Frag {
  v8i fb[C::NB];     // B tile rows (MFMA A operand)
  v8i fa[C::MB];     // A tile rows (MFMA B operand)
  float sam[C::MB];  // A scale of this lane's row in each 16-row block
  float sbn[C::NB][4];  // row mode: B scales of this lane's 4 columns per block
  float sbv;            // block mode: the wave's B block scale
};

// `slot` is the scale-ring slot holding the group, `gq` the group's index
// inside its scale block.
template <class C, bool BROW>
__device__ __forceinline__ void load_frag(Frag<C>& f, const uint8_t* stage, const float* slot, int gq,
                                          int wm, int wn, int lane) {
  const uint8_t* la = stage;
  const uint8_t* lb = stage + C::A_BYTES;
  const float* lsb = slot + C::SA_BYTES / 4;
  const int fr = lane & 15;
  const int kc = lane >> 4;  // k chunks kc and kc + 4 (any permutation shared by A and B is valid)
#pragma unroll
  for (int j = 0; j < C::NB; ++j) {
    const int r = (wn * C::NB + j) * 16 + fr;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(lb + swz(r, kc));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(lb + swz(r, kc + 4));
    f.fb[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
    const int rb = wm * C::MB + i;
    const int r = rb * 16 + fr;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(la + swz(r, kc));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(la + swz(r, kc + 4));
    f.fa[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    f.sam[i] = slot[(rb * SBLK + gq) * 16 + fr];
  }
  if (BROW) {
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(lsb + ((wn * C::NB + j) * SBLK + gq) * 16 + 4 * kc);
      f.sbn[j][0] = v.x; f.sbn[j][1] = v.y; f.sbn[j][2] = v.z; f.sbn[j][3] = v.w;
    }
  } else {
    f.sbv = lsb[gq * 16 + (wn * C::NB * 16) / 128];
  }
}

// Software-pipelined K group for the three-stage path.  The MFMAs of the
// current group are issued one per step; each step also promotes the
// partial of the MFMA issued LAG steps earlier, issues one read of the next
// group's fragments from LDS, and every other step one global -> LDS copy,
// so the LDS and the load unit see a steady stream instead of a burst
// after each barrier.  A scheduling barrier after every step keeps that
// placement.
// LAG is a template parameter of the group: 3 for BF16 or FP32 output with
// block scales (1-1.5% faster than 2 at 4096 x 18432 x 7168 and on the
// K = 2048 shapes), 2 for row scales (3 was 3% slower there) and the
// quantized output (3 spills there).  The promotion order is the same for
// every lag, so the results are too.

// Read number k of the next group's fragments: B rows, A rows, A scales,
// then the B scales.
template <class C, bool BROW>
__device__ __forceinline__ void read_op(Frag<C>& f, int k, const uint8_t* stage, const float* slot,
                                        int gq, int wm, int wn, int lane) {
  const uint8_t* la = stage;
  const uint8_t* lb = stage + C::A_BYTES;
  const float* lsb = slot + C::SA_BYTES / 4;
  const int fr = lane & 15;
  const int kc = lane >> 4;
  if (k < C::NB) {
    const int r = (wn * C::NB + k) * 16 + fr;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(lb + swz(r, kc));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(lb + swz(r, kc + 4));
    f.fb[k] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  } else if (k < C::NB + C::MB) {
    const int i = k - C::NB;
    const int r = (wm * C::MB + i) * 16 + fr;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(la + swz(r, kc));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(la + swz(r, kc + 4));
    f.fa[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  } else if (k < C::NB + 2 * C::MB) {
    const int i = k - C::NB - C::MB;
    f.sam[i] = slot[((wm * C::MB + i) * SBLK + gq) * 16 + fr];
  } else if (BROW) {
    const int j = k - C::NB - 2 * C::MB;
    const float4 v = *reinterpret_cast<const float4*>(lsb + ((wn * C::NB + j) * SBLK + gq) * 16 + 4 * kc);
    f.sbn[j][0] = v.x; f.sbn[j][1] = v.y; f.sbn[j][2] = v.z; f.sbn[j][3] = v.w;
  } else {
    f.sbv = lsb[gq * 16 + (wn * C::NB * 16) / 128];
  }
}

template <class C, bool BROW>
constexpr int read_ops() { return C::NB + 2 * C::MB + (BROW ? C::NB : 1); }

template <class C, bool BROW>
__device__ __forceinline__ void promote(v4f (&acc)[C::MB][C::NB], const v4f& part, int s,
                                        const Frag<C>& f) {
  const int i = s / C::NB, j = s % C::NB;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float sc = BROW ? f.sam[i] * f.sbn[j][q] : f.sam[i] * f.sbv;
    acc[i][j][q] = __builtin_fmaf(part[q], sc, acc[i][j][q]);
  }
}

// issue_part(k) issues copy k of the next issue (k < copies).
template <class C, bool BROW, int COPIES, int LAG, class IssuePart>
__device__ __forceinline__ void pipelined_group(v4f (&acc)[C::MB][C::NB], const Frag<C>& cur,
                                                Frag<C>& nxt, const uint8_t* stage_n,
                                                const float* slot_n, int gq_n, int wm, int wn,
                                                int lane, IssuePart&& issue_part) {
  constexpr int S = C::MB * C::NB;
  constexpr int NR = read_ops<C, BROW>();
  static_assert(S >= 2, "steps");
  v4f part[S];
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int s = 0; s < S + LAG; ++s) {
    if (s < S) part[s] = mfma_16x16x128_fp8(cur.fb[s % C::NB], cur.fa[s / C::NB]);
    if (s >= LAG) promote<C, BROW>(acc, part[s - LAG], s - LAG, cur);
    // reads k in [s NR / S, (s + 1) NR / S); copies spread over steps 1 .. S - 1
    if (s < S) {
#pragma unroll
      for (int k = s * NR / S; k < (s + 1) * NR / S; ++k)
        read_op<C, BROW>(nxt, k, stage_n, slot_n, gq_n, wm, wn, lane);
    }
    if (s >= 1 && s < S) {
#pragma unroll
      for (int k = (s - 1) * COPIES / (S - 1); k < s * COPIES / (S - 1); ++k) issue_part(k);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Output forms of the epilogue.
constexpr int kOutBf16 = 0;  // BF16, nearest-even
constexpr int kOutF32 = 1;   // FP32
constexpr int kOutFp8 = 2;   // E4M3 codes + one FP32 scale per 1x128 tile along N

template <class C, int OUT, bool BROW, bool GROUPED>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmArgs p) {
  constexpr int BM = C::BM, BN = C::BN;
  static_assert(C::lds_bytes(BROW) <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) uint8_t lds[C::lds_bytes(BROW)];
  poison_lds<C::lds_bytes(BROW)>(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int G = static_cast<int>(p.K / 128);

  // ---- tiles: the workgroup walks the virtual workgroup ids blockIdx.x,
  //      blockIdx.x + gridDim.x, ... (gridDim.x is a multiple of the XCD
  //      count, so every tile of a workgroup maps to the same XCD).
  //      plan_tile(v, ...) gives virtual tile v's first row, row end, first
  //      column and its expert's B and B scales (false: no such tile).
  //      The grouped form's host-side M-tile count is an upper bound (the
  //      offsets are on the device), so the kernel counts the experts' tiles
  //      itself: with the bound, the empty virtual tiles (up to E per tile
  //      column) would all fall on the last XCD, and the chunked order would
  //      give whole empty rounds.
  int64_t m0 = 0, m_end = 0, n0 = 0;
  const uint8_t* bmat = p.b;
  const float* sbmat = p.sb;
  auto expert_rows = [&](int e, int64_t& r0, int64_t& r1) {
    // offsets are clamped into [0, M] so that inconsistent offsets can only
    // give wrong rows, never an out-of-bounds access
    r0 = p.offsets[e];
    r1 = p.offsets[e + 1];
    r0 = r0 < 0 ? 0 : (r0 > p.M ? p.M : r0);
    r1 = r1 < r0 ? r0 : (r1 > p.M ? p.M : r1);
  };
  int tiles_m = p.tiles_m;
  if (GROUPED) {
    int64_t tm = 0;
    for (int e = 0; e < p.E; ++e) {
      int64_t r0, r1;
      expert_rows(e, r0, r1);
      tm += (r1 - r0 + BM - 1) / BM;
    }
    // never above the bound (which the launch checked against int range)
    tiles_m = static_cast<int>(tm < p.tiles_m ? tm : p.tiles_m);
  }
  // grouped: whole chunk rounds of virtual ids (a multiple of 8 kChunk
  // within the launch's int range, which the bound's tile count leaves)
  const int vtiles = GROUPED ? static_cast<int>((static_cast<int64_t>(tiles_m) * p.tiles_n + NUM_XCD * kChunk - 1) /
                                                (NUM_XCD * kChunk) * (NUM_XCD * kChunk))
                             : tiles_m * p.tiles_n;
  auto plan_tile = [&](int v, int64_t& m0, int64_t& m_end, int64_t& n0, const uint8_t*& bmat,
                       const float*& sbmat) -> bool {
    int vm, nt;
    if (GROUPED) {
      if (!tile_of_chunked(v, tiles_m, p.tiles_n, vm, nt)) return false;
    } else {
      tile_of<GROUP_M>(v, tiles_m, p.tiles_n, vm, nt);
    }
    n0 = static_cast<int64_t>(nt) * BN;
    bmat = p.b;
    sbmat = p.sb;
    if (GROUPED) {
      int64_t mt = vm;
      for (int e = 0; e < p.E; ++e) {
        int64_t r0, r1;
        expert_rows(e, r0, r1);
        const int64_t tiles = (r1 - r0 + BM - 1) / BM;
        if (mt < tiles) {
          m0 = r0 + mt * BM;
          m_end = r1;
          bmat = p.b + static_cast<int64_t>(e) * p.N * p.K;
          sbmat = p.sb + static_cast<int64_t>(e) * ((p.N + 127) / 128) * G;
          return true;
        }
        mt -= tiles;
      }
      return false;
    }
    m0 = static_cast<int64_t>(vm) * BM;
    m_end = p.M;
    return true;
  };
  // block mode: a wave's columns lie inside one 128-wide block of B
  static_assert(BROW || (128 % (C::NB * 16) == 0), "wave columns must not straddle a B block");

  // ---- tile copy plan: the tile rows of a K group are DPW 1 KiB copies per
  //      wave; copy q of wave w moves rows 8 (q NW + w) .. 8 (q NW + w) + 7
  //      of the tile pair (A rows first, then B rows), so whether it is an A
  //      or a B copy depends on q only, and its rows are the wave's rows of
  //      copy 0 moved by a multiple of 8 NW rows (a uniform offset).  Lane l
  //      fetches the global chunk (l & 7) ^ swizzle(row) of row l / 8 of its
  //      copy; the swizzle does not depend on q.  The buffer descriptors
  //      (per tile) cover the tile's valid rows.
  static_assert((BM / 8) % C::NW == 0 && C::NW % 2 == 0, "A copies must be whole rounds over the waves");
  constexpr int QA = BM / 8 / C::NW;  // copies per wave that move A rows
  const uint32_t lda = static_cast<uint32_t>(p.lda), ldb = static_cast<uint32_t>(p.ldb);
  uint32_t voff[C::DPW];  // copy k: its rows' offsets from the tile's first row
  {
    const int r = 8 * wave + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
#pragma unroll
    for (int k = 0; k < C::DPW; ++k)
      voff[k] = k < QA ? static_cast<uint32_t>(r + k * 8 * C::NW) * lda + c * 16
                       : static_cast<uint32_t>(r + (k - QA) * 8 * C::NW) * ldb + c * 16;
  }
  i32x4 rs_a, rs_b;

  // ---- scale copy plan: every issue copies one quarter of a scale block
  //      (SBLK groups).  The quarter is split into units of 16 rows x SBLK
  //      groups, one dword copy each: SAW units of A scales, then SBW units
  //      of B scales (row mode: 16 rows each; block mode: all the tile's
  //      128-row blocks).  Wave w issues units w, w + NW, ... (SPW per
  //      wave); units past the last re-read a valid A scale into a dummy
  //      LDS area.  A-scale unit c, quarter q covers rows 16 (q SAW + c) ..
  //      + 15 (lane l: row + l % 16, group SBLK h + l / 16).
  constexpr int SAW = C::SAW, SBW = C::sbw(BROW);
  constexpr int SPW = (SAW + SBW + C::NW - 1) / C::NW;  // scale copies per wave per issue
  struct ScaleCopy {
    i32x4 rs;
    uint32_t voff, qstep, hstep, dst0, dstq, slot;
  };
  ScaleCopy sc[SPW];
  const uint32_t ldsa4 = static_cast<uint32_t>(p.ldsa * 4), ldsb4 = static_cast<uint32_t>(p.ldsb * 4);
  // VGPR offset of this wave's scale copy u for lane index ln
  auto scale_voff = [&](int u, int ln) -> uint32_t {
    const int c = wave + u * C::NW;
    const uint32_t gl = static_cast<uint32_t>(ln >> 4) * 4u;
    if (c < SAW) return static_cast<uint32_t>(16 * c + (ln & 15)) * ldsa4 + gl;
    if (c < SAW + SBW) {
      const int w = c - SAW;
      return BROW ? static_cast<uint32_t>(16 * w + (ln & 15)) * ldsb4 + gl
                  : static_cast<uint32_t>(ln & 15) * ldsb4 + gl;
    }
    return 0;
  };
  {
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int c = wave + u * C::NW;
      ScaleCopy& x = sc[u];
      x.hstep = SBLK * 4;
      x.slot = C::slot_bytes(BROW);
      x.voff = scale_voff(u, lane);
      if (c < SAW) {
        x.qstep = 16 * SAW * ldsa4;
        x.dst0 = c * 256;
        x.dstq = SAW * 256;
      } else if (c < SAW + SBW) {
        const int w = c - SAW;
        if (BROW) {
          x.qstep = 16 * SBW * ldsb4;
          x.dst0 = C::SA_BYTES + w * 256;
          x.dstq = SBW * 256;
        } else {
          x.qstep = 0;
          x.dst0 = C::SA_BYTES;
          x.dstq = 0;
        }
      } else {
        x.qstep = 0;
        x.hstep = 0;
        x.dst0 = C::dummy_off(BROW) - C::sc_area();
        x.dstq = 0;
        x.slot = 0;
      }
    }
  }
  // per-tile descriptors: A and B rows, A scales, B scales
  struct TileDesc {
    i32x4 a, b, sa, sb;
  };
  auto descriptors = [&](int64_t m0, int64_t m_end, int64_t n0, const uint8_t* bmat,
                         const float* sbmat) -> TileDesc {
    const int64_t rows_a = m_end - m0 < BM ? m_end - m0 : BM;
    const int64_t rows_b = p.N - n0 < BN ? p.N - n0 : BN;
    TileDesc d;
    d.a = make_rsrc(p.a + m0 * p.lda, static_cast<uint32_t>(rows_a * p.lda));
    d.b = make_rsrc(bmat + n0 * p.ldb, static_cast<uint32_t>(rows_b * p.ldb));
    d.sa = make_rsrc(p.sa + m0 * p.ldsa, static_cast<uint32_t>(rows_a) * ldsa4);
    if (BROW) {
      d.sb = make_rsrc(sbmat + n0 * p.ldsb, static_cast<uint32_t>(rows_b) * ldsb4);
    } else {
      const int64_t blocks = (rows_b + 127) / 128;
      d.sb = make_rsrc(sbmat + (n0 / 128) * p.ldsb, static_cast<uint32_t>(blocks) * ldsb4);
    }
    return d;
  };
  // whether this wave's scale copy u moves B scales (else A scales, or a
  // dummy copy of A scales)
  auto copies_sb = [&](int u) {
    const int c = wave + u * C::NW;
    return c >= SAW && c < SAW + SBW;
  };
  auto set_tile_copies = [&](const TileDesc& d) {
    rs_a = d.a;
    rs_b = d.b;
#pragma unroll
    for (int u = 0; u < SPW; ++u) sc[u].rs = copies_sb(u) ? d.sb : d.sa;
  };
  // descriptor k of the next tile's record in LDS, made uniform
  auto next_desc = [&](int k) -> i32x4 {
    const i32x4 d = *reinterpret_cast<const i32x4*>(lds + C::next_off(BROW) + 16 * k);
    i32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __builtin_amdgcn_readfirstlane(d[e]);
    return r;
  };

  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds[0]));
  constexpr int COPIES = C::DPW + SPW;  // vector-memory ops per wave per issue
  constexpr int SLOT = C::slot_bytes(BROW);

  // this wave's copy u of quarter q of scale block h
  // (hs = h % NSLOT, passed separately so that it can be a constant).  The
  // quarter's row offset and the block's group offset are added to the
  // VGPR offset, so the descriptor's range check covers the whole address
  // (the SGPR offset stays zero).
  auto issue_scales_v = [&](int u, uint32_t voff, int q, int h, int hs) {
    const ScaleCopy& x = sc[u];
    const uint32_t dst = lds_base + C::sc_area() + hs * x.slot + x.dst0 + x.dstq * q;
    gemm_copy4(x.rs, voff + x.qstep * q + x.hstep * h, 0, dst);
  };
  auto issue_scales = [&](int u, int q, int h, int hs) { issue_scales_v(u, sc[u].voff, q, h, hs); };
  // part k of issue t: tile copy k (k < DPW) of K group min(t, G - 1) into
  // `stage`, or (k >= DPW) copy k - DPW of quarter t % 4 of scale block
  // t / 4 + 1 (block 0 is copied with the first two issues)
  auto issue_part = [&](int t, int stage, int k) {
    const uint32_t gk = static_cast<uint32_t>(t < G - 1 ? t : G - 1) * 128u;
    const uint32_t base = lds_base + stage * C::STAGE;
    if (k < QA)
      gemm_copy16(rs_a, voff[k], gk, base + (k * C::NW + wave) * 1024);
    else if (k < C::DPW)
      gemm_copy16(rs_b, voff[k], gk, base + C::A_BYTES + ((k - QA) * C::NW + wave) * 1024);
    else
      issue_scales(k - C::DPW, t & 3, (t >> 2) + 1, ((t >> 2) + 1) % NSLOT);
  };
  // the same with the issue's quarter and scale slot given (constants in
  // the unrolled loop)
  auto issue_part_q = [&](int t, int stage, int q, int h, int hs, int k) {
    const uint32_t gk = static_cast<uint32_t>(t < G - 1 ? t : G - 1) * 128u;
    const uint32_t base = lds_base + stage * C::STAGE;
    if (k < QA)
      gemm_copy16(rs_a, voff[k], gk, base + (k * C::NW + wave) * 1024);
    else if (k < C::DPW)
      gemm_copy16(rs_b, voff[k], gk, base + C::A_BYTES + ((k - QA) * C::NW + wave) * 1024);
    else
      issue_scales(k - C::DPW, q, h, hs);
  };
  auto issue = [&](int t, int stage) {
#pragma unroll
    for (int k = 0; k < COPIES; ++k) issue_part(t, stage, k);
  };
  // the copies a tile needs before its first barrier: scale block 0 and
  // issues 0 and 1
  // (with scale offsets made here: kept from the set-up they are spilled
  // around the epilogue, and each reload would wait for the copies before)
  auto issue_head = [&]() {
    const int hl = opaque_lane();
    uint32_t vb[SPW];
#pragma unroll
    for (int u = 0; u < SPW; ++u) vb[u] = scale_voff(u, hl);
#pragma unroll
    for (int q = 0; q < SBLK; ++q)
#pragma unroll
      for (int u = 0; u < SPW; ++u) issue_scales_v(u, vb[u], q, 0, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int k = 0; k < COPIES; ++k) {
        if (k < C::DPW) issue_part(t, t, k);
        else issue_scales_v(k - C::DPW, vb[k - C::DPW], t & 3, 1, 1 % NSLOT);
      }
  };
  auto slot_of = [&](int g) {
    return reinterpret_cast<const float*>(lds + C::sc_area() + ((g / SBLK) % NSLOT) * SLOT);
  };

  // Tile stream.  When G is a multiple of SBLK and at least 8, tile
  // boundaries fall on scale-block boundaries, and a tile's last issues copy
  // its successor's first scale block (issues G - 4 .. G - 1) and first
  // three K groups (issues G .. G + 2); its last iteration reads the
  // successor's first fragments.  The successor then starts with no head
  // copies and no wait: only the output tile goes through LDS in between.
  // Stages, scale slots and fragment sets then follow the workgroup's
  // running group count u (tile k's group g has u = k G + g): stage u % 3,
  // slot (u / 4) % 3, set u % 2.  j0 = (k G) % 12 (0, 4 or 8) is the
  // phase of a tile's group 0 in that period-12 pattern; the unrolled loop
  // runs rounds of 12 values of u, so every index stays a constant.  At the
  // two switch points the copies take the successor's descriptors, which
  // the tile start leaves in LDS.  Otherwise (and for a workgroup's first
  // tile) the head copies are issued after the last group, j0 = 0.  The
  // quantized output keeps the head: its epilogue (FP32 staging and the
  // encoder) with a fragment set held across it spills, and measured
  // slower than without the stream (544 against 517 us at 4096 x 18432 x
  // 7168).
  const bool streamable = OUT != kOutFp8 && G % SBLK == 0 && G >= 8;
  const int nblk = G / SBLK;  // scale blocks per tile (when streamable)

  int v = blockIdx.x;
  while (v < vtiles && !plan_tile(v, m0, m_end, n0, bmat, sbmat)) v += gridDim.x;
  if (v >= vtiles) return;  // uniform per workgroup
  set_tile_copies(descriptors(m0, m_end, n0, bmat, sbmat));
  issue_head();

  bool head = true;
  int j0 = 0;
  // Fragment set f0 carries the next tile's group 0 across the epilogue.
  // Every tile starts at an even position (j0 is 0, 4 or 8), which reads f0
  // and fills f1, so f1 starts each tile unset and holds nothing across.
  Frag<C> f0;
  for (;;) {
    Frag<C> f1;
    // ---- the workgroup's next tile; its descriptors go to LDS for the
    //      switch points (read there after at least one barrier)
    int vn = v + gridDim.x;
    {
      int64_t nm0, nm_end, nn0;
      const uint8_t* nb;
      const float* nsb;
      while (vn < vtiles && !plan_tile(vn, nm0, nm_end, nn0, nb, nsb)) vn += gridDim.x;
      if (streamable && vn < vtiles && tid == 0) {
        const TileDesc d = descriptors(nm0, nm_end, nn0, nb, nsb);
        i32x4* rec = reinterpret_cast<i32x4*>(lds + C::next_off(BROW));
        rec[0] = d.a;
        rec[1] = d.b;
        rec[2] = d.sa;
        rec[3] = d.sb;
      }
    }
    const bool more = vn < vtiles;
    const bool pre = streamable && more;  // this tile prefetches the next one

    v4f acc[C::MB][C::NB];
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Pipeline over three stages.  Before iteration g: fragments of group
    // g are in registers (cur), the stage of group g + 1 holds it and is
    // visible, the copy of group g + 2 is in flight.  Iteration g reads the
    // fragments of g + 1, starts issue g + 3 into the stage of group g
    // (whose reads finished before the last barrier), multiplies g, then
    // waits for issue g + 2 and for its own LDS reads before the barrier.
    // Scale block h is copied by issues 4h - 4 .. 4h - 1 (iterations
    // 4h - 7 .. 4h - 4), is first read in iteration 4h - 1, and its slot
    // (NSLOT = 3) was last read in iteration 4h - 10.  Without a successor
    // to prefetch, copies and reads past the last group are clamped to
    // valid data that is never used.
    if (head) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this tile's head copies (and earlier stores)
      block_barrier();
      load_frag<C, BROW>(f0, lds, slot_of(0), 0, wm, wn, opaque_lane());  // addresses made here, not reloaded
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      issue(2, 2);
      block_barrier();
    }

    // Unrolled by 12 (fragment sets alternate with period 2, stages with 3,
    // scale quarters with 4, scale slots with 12) so that every stage, slot
    // and quarter index is a constant; iteration g + i runs only if
    // 0 <= g + i < G.  Issues past the last group copy from the successor
    // once the switch points have passed (gsub, hsub: its group and block
    // numbers are those of this tile minus G and nblk).
    int gsub = 0, hsub = 0;
    for (int g = -j0; g < G; g += 12) {
      const int hb = g / 4;  // scale blocks before this round (g is a multiple of 4)
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        if (static_cast<unsigned>(g + i) < static_cast<unsigned>(G)) {
          Frag<C>& cur = (i & 1) ? f1 : f0;
          Frag<C>& nxt = (i & 1) ? f0 : f1;
          const int t = g + i + 3;                   // this iteration's issue
          const int q = (i + 3) & 3;                 // its scale quarter
          const int hl = (i + 3) / 4 + 1;            // its scale block, minus hb
          // G + j0 is a multiple of 4, so both switch points (issues G - 4
          // and G, iterations G - 7 and G - 3) fall where i % 4 == 1
          if ((i & 3) == 1 && pre) {
            if (t == G - 4) {
#pragma unroll
              for (int u = 0; u < SPW; ++u) sc[u].rs = next_desc(copies_sb(u) ? 3 : 2);
              hsub = nblk;
            } else if (t == G) {
              rs_a = next_desc(0);
              rs_b = next_desc(1);
              gsub = G;
            }
          }
          const float* slot_n = reinterpret_cast<const float*>(
              lds + C::sc_area() + (((i + 1) / 4) % NSLOT) * SLOT);  // group g + i + 1
          pipelined_group<C, BROW, COPIES, (BROW || OUT == kOutFp8) ? 2 : 3>(
              acc, cur, nxt, lds + ((i + 1) % 3) * C::STAGE, slot_n, (i + 1) & 3, wm, wn, lane,
              [&](int k) { issue_part_q(t - gsub, i % 3, q, hb + hl - hsub, hl % NSLOT, k); });
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(COPIES));
          __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
          block_barrier();
        }
      }
    }

    // ---- the next tile becomes current; without the stream its head
    //      copies go out before this tile's results
    const int64_t cm0 = m0, cm_end = m_end, cn0 = n0;
    if (more) plan_tile(vn, m0, m_end, n0, bmat, sbmat);
    if (!pre) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the clamped copies past the last group
      block_barrier();                            // every stage and scale slot is free
      if (more) {
        set_tile_copies(descriptors(m0, m_end, n0, bmat, sbmat));
        issue_head();
      }
    }

    // ---- epilogue through a free stage of the LDS (the stage of the next
    //      tile's group 0, read out in the last iteration, or stage 2 after
    //      head copies into stages 0 and 1), padded rows, PR rows per pass,
    //      so that every global store writes 16 contiguous bytes per lane
    //      and a wave writes whole output rows.  Lane (fr, kc) holds
    //      columns 4 kc .. 4 kc + 3 of row fr of each 16x16 block.  The
    //      stores carry the non-temporal hint: the kernel never reads its
    //      output, and the caches stay with the operand panels.
    constexpr int OB = OUT == kOutBf16 ? 2 : 4;   // staged bytes per element
    constexpr int ROWB = BN * OB + 16;            // padded LDS row
    constexpr int CPR = BN * OB / 16;             // 16-byte chunks per tile row
    constexpr int PR0 = C::STAGE / ROWB;          // rows that fit one stage
    constexpr int PR = PR0 >= BM ? BM : PR0 >= 128 ? 128 : PR0 >= 64 ? 64 : PR0 >= 32 ? 32 : 16;
    static_assert(PR <= PR0 && BM % PR == 0, "output passes");
    uint8_t* const ob = lds + (pre ? (j0 + G) % 3 : 2) * C::STAGE;
    uint8_t* dbase = static_cast<uint8_t*>(p.d);
    const int64_t ldd_b = p.ldd * OB;
    const int64_t cols = p.N - cn0 < BN ? p.N - cn0 : BN;   // valid columns of the tile
    // a whole tile whose pass fits 32-bit lane offsets (uniform)
    const bool full = cols == BN && cm_end - cm0 >= BM && ldd_b * PR < (int64_t(1) << 31);
    // The lane addresses below come from a lane index made where each part
    // uses it (opaque_lane): hoisted out of the tile loop, or carried across
    // the passes, they would be spilled, and each reload from scratch waits
    // for every copy and store in flight.
#pragma unroll
    for (int pass = 0; pass < BM / PR; ++pass) {
      if (pass > 0) block_barrier();  // previous pass read out of the LDS
      {
        const int elane = opaque_lane();
        const int fr = elane & 15;
        const int kc = elane >> 4;
#pragma unroll
        for (int i = 0; i < C::MB; ++i) {
          const int rb = wm * (C::MB * 16) + i * 16;  // first row of the block
          if (rb / PR != pass) continue;              // uniform
          const int r = rb % PR + fr;
#pragma unroll
          for (int j = 0; j < C::NB; ++j) {
            const int c = wn * (C::NB * 16) + j * 16 + 4 * kc;
            const v4f vv = acc[i][j];
            uint8_t* dst = ob + r * ROWB + c * OB;
            if (OUT != kOutBf16) {
              *reinterpret_cast<float4*>(dst) = make_float4(vv[0], vv[1], vv[2], vv[3]);
            } else {
              *reinterpret_cast<uint2*>(dst) =
                  make_uint2(pack_bf16x2_rne(vv[0], vv[1]), pack_bf16x2_rne(vv[2], vv[3]));
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);  // this wave's LDS writes are done
      block_barrier();
      if (OUT == kOutFp8) {
        // quantize the staged FP32 rows as 1x128 tiles along N: one 16-lane
        // DPP row per tile, 8 values per lane, every lane active for the
        // row max-abs; tiles past M or N are computed and not stored
        constexpr int GPR = BN / 128;                // tiles per tile row
        constexpr int UNITS = PR * GPR;
        static_assert(UNITS % (C::NT / 16) == 0, "quantized output passes");
        const int sub = lane & 15;
        uint8_t* const qbase = static_cast<uint8_t*>(p.d);
#pragma unroll
        for (int u0 = 0; u0 < UNITS; u0 += C::NT / 16) {
          const int u = u0 + (tid >> 4);
          const int r = u / GPR, gc = u % GPR;
          const float* src = reinterpret_cast<const float*>(ob + r * ROWB + (gc * 128 + sub * 8) * 4);
          const float4 x0 = *reinterpret_cast<const float4*>(src);
          const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
          const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          float am = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
          am = row16_max(am);
          const TileScale ts = make_tile_scale(am);
          const uint2 cw = make_uint2(encode4(v, ts), encode4(v + 4, ts));
          const int64_t m = cm0 + pass * PR + r;
          const int c0 = gc * 128;
          if (m < cm_end && c0 < cols) {
            __builtin_nontemporal_store(u32x2{cw.x, cw.y},
                                        reinterpret_cast<u32x2*>(qbase + m * p.ldd + cn0 + c0 + sub * 8));
            if (sub == 0) p.s_out[m * p.lds_out + (cn0 + c0) / 128] = ts.s;
          }
        }
      } else if (full) {
        // a whole tile: no bounds, one base address per pass
        static_assert((PR * CPR) % C::NT == 0, "whole store rounds");
        uint8_t* const tb = dbase + (cm0 + pass * PR) * ldd_b + cn0 * OB;
        const int et = wave * 64 + opaque_lane();
#pragma unroll
        for (int k = 0; k < PR * CPR / C::NT; ++k) {
          const int ch = et + k * C::NT;
          const int r = ch / CPR, cc = ch % CPR;
          const uint4 vv = *reinterpret_cast<const uint4*>(ob + r * ROWB + cc * 16);
          const uint32_t off = static_cast<uint32_t>(r) * static_cast<uint32_t>(ldd_b) + cc * 16;
          __builtin_nontemporal_store(u32x4{vv.x, vv.y, vv.z, vv.w}, reinterpret_cast<u32x4*>(tb + off));
        }
      } else {
        const int et = wave * 64 + opaque_lane();
  #pragma unroll 4
        for (int ch = et; ch < PR * CPR; ch += C::NT) {
          const int r = ch / CPR, cc = ch % CPR;
          const int64_t m = cm0 + pass * PR + r;
          const int c0 = cc * (16 / OB);
          if (m >= cm_end || c0 >= cols) continue;
          const uint4 vv = *reinterpret_cast<const uint4*>(ob + r * ROWB + cc * 16);
          uint8_t* dst = dbase + m * ldd_b + (cn0 + c0) * OB;
          if (c0 + 16 / OB <= cols) {
            __builtin_nontemporal_store(u32x4{vv.x, vv.y, vv.z, vv.w}, reinterpret_cast<u32x4*>(dst));
          } else {
            // the row's last columns: byte by byte from the chunk's words
            const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
            const int nb = static_cast<int>(cols - c0) * OB;
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (e < nb) dst[e] = static_cast<uint8_t>(w[e >> 2] >> (8 * (e & 3)));
          }
        }
      }
    }
    if (!more) break;
    if (pre) block_barrier();  // the staged output is read out before its stage takes group 3
    v = vn;
    head = !pre;
    j0 = pre ? (j0 + G) % 12 : 0;
  }
}

template <class C, bool BROW, bool GROUPED>
hipError_t dispatch(GemmArgs args, int64_t tiles_m_extra, int out, hipStream_t st) {
  const int64_t tm = (args.M + C::BM - 1) / C::BM + tiles_m_extra, tn = (args.N + C::BN - 1) / C::BN;
  // (room left for the grouped order's rounding to whole chunk rounds)
  if (tm * tn > 0x7fffffff - NUM_XCD * kChunk) return hipErrorInvalidValue;
  args.tiles_m = static_cast<int32_t>(tm);
  args.tiles_n = static_cast<int32_t>(tn);
  // persistent: one workgroup per compute unit of a 256-CU MI355X (a
  // multiple of the XCD count), each walking tiles gridDim.x apart
  const int64_t vt = tm * tn;
  const dim3 grid(static_cast<unsigned>(vt < kGridCap ? vt : kGridCap)), block(C::NT);
  if (out == kOutF32) hipLaunchKernelGGL((gemm_kernel<C, kOutF32, BROW, GROUPED>), grid, block, 0, st, args);
  else if (out == kOutFp8) {
    // not offered for the grouped form, nor for block scales on the small
    // tiles (block-scale problems take 128x256 tiles with this output)
    if constexpr (GROUPED || (!BROW && C::BN != 256)) return hipErrorInvalidValue;
    else hipLaunchKernelGGL((gemm_kernel<C, kOutFp8, BROW, GROUPED>), grid, block, 0, st, args);
  }
  else hipLaunchKernelGGL((gemm_kernel<C, kOutBf16, BROW, GROUPED>), grid, block, 0, st, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const float* sa, int64_t lda, int64_t ldsa,
                       const uint8_t* b, const float* sb, int64_t ldb, int64_t ldsb,
                       bool bscale_row, void* d, int64_t ldd, float* s_out, int64_t lds_out,
                       int out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  GemmArgs args{};
  args.a = a; args.sa = sa; args.b = b; args.sb = sb; args.d = d; args.offsets = nullptr;
  args.s_out = s_out; args.lds_out = lds_out;
  args.lda = lda; args.ldsa = ldsa; args.ldb = ldb; args.ldsb = ldsb; args.ldd = ldd;
  args.M = M; args.N = N; args.K = K; args.E = 0;
  if (bscale_row) return dispatch<RowCfg, true, false>(args, 0, out, st);
  const int64_t small_tiles = (M + SmallCfg::BM - 1) / SmallCfg::BM * ((N + SmallCfg::BN - 1) / SmallCfg::BN);
  if (out != kOutFp8 && small_tiles <= kGridCap) return dispatch<SmallCfg, false, false>(args, 0, out, st);
  return dispatch<MainCfg, false, false>(args, 0, out, st);
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
  return dispatch<MainCfg, false, true>(args, E, out_f32 ? kOutF32 : kOutBf16, st);
}

}  // namespace fp8bs
