/*
 * fp8bs.h -- C ABI of libfp8bs: fine-grained FP8 quantization and the
 * block-scaled FP8 GEMM on AMD Instinct MI355X (gfx950).
 *
 * The method is the fine-grained FP8 scheme of the DeepSeek-V3 report
 * excerpts on five web pages, cited as
 *   [p1] xn--9g3bo1gtkw0l8ubf92bgle.kr board post wr_id=32373
 *   [p2] why-be.why-be.co.kr board post wr_id=73620
 *   [p3] xn--9g3bo1gtkw0l8ubf92bgle.kr board post wr_id=113503
 *   [p4] bestpmk.kr board post wr_id=299512
 * with a paragraph number counted on that page.
 *
 * Number formats (readings adopted where the pages only say "FP8"):
 *   - codes are OCP E4M3FN bytes (bias 7, largest finite 448, NaN 0x7F/0xFF,
 *     no infinities), the byte layout of torch.float8_e4m3fn;
 *   - every scale is an IEEE binary32 value s = fl32(amax / 448) of the
 *     max-abs of its tile; a code is the nearest-even E4M3 value of the
 *     exact quotient x / s, saturated to +-448; an all-zero tile has s = 0
 *     and signed-zero codes; subnormal scales are kept (no flush to zero);
 *   - the value a code stands for is dec(code) * s.
 * Inputs must be finite; NaN or infinite inputs give unspecified codes.
 *
 * Conventions for every entry point:
 *   - All buffers are device memory owned by the caller; the library keeps
 *     no pointer after the call returns and allocates nothing.
 *   - Element strides ("ld") are counted in elements of the buffer's type
 *     and are row strides of row-major matrices.
 *   - Byte buffers (codes, bf16, fp32 matrices) must be 16-byte aligned and
 *     their row strides a multiple of 16 bytes; scale buffers must be 4-byte
 *     aligned and may have any stride at least the row length.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the null
 *     stream) and runs asynchronously; no call synchronizes with the host.
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns an error and enqueues nothing.  A launch failure returns
 *     FP8BS_ERR_LAUNCH.  Calls are thread-safe.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8BS_OK = 0,
    FP8BS_ERR_INVALID_ARG = 1,      /* null pointer, negative size, bad enum, stride too small */
    FP8BS_ERR_UNSUPPORTED_SHAPE = 2,/* K (or C) not a multiple of 128 */
    FP8BS_ERR_MISALIGNED = 3,       /* pointer or row stride breaks the alignment rules */
    FP8BS_ERR_NO_DEVICE = 4,        /* no HIP device, or the device is not gfx950 */
    FP8BS_ERR_LAUNCH = 5            /* the kernel launch failed */
} fp8bs_status;

typedef enum { FP8BS_OUT_BF16 = 0, FP8BS_OUT_F32 = 1 } fp8bs_out_dtype;

typedef enum {
    FP8BS_BSCALE_BLOCK_128x128 = 0, /* sb[(n/128)*ldsb + k/128]: weight blocks */
    FP8BS_BSCALE_ROW_1x128 = 1      /* sb[n*ldsb + k/128]: 1x128 tiles along K */
} fp8bs_bscale;

typedef enum {
    FP8BS_SRC_FP8_1x128 = 0,        /* E4M3 codes with 1x128 scales */
    FP8BS_SRC_BF16 = 1,             /* plain bf16 */
    FP8BS_SRC_E5M6 = 2              /* 12-bit E5M6 rows as fp8bs_encode_e5m6 packs them */
} fp8bs_requant_src;

/*
 * Activation quantization with 1x128 tiles along K.
 * [p1] para 3: the max-abs is taken online for every 1x128 activation tile,
 * a scaling factor is derived from it and the tile is quantized to FP8;
 * [p1] para 2: the scales are per group along the inner dimension K.
 *   x  bf16 [M][ldx]            input, row m holds K values
 *   q  u8   [M][ldq]            E4M3 codes
 *   s  f32  [M][lds]            s[m*lds + g] scales tile (m, g), g < K/128
 * M >= 0 (0 is a no-op), K > 0 and K % 128 == 0.
 */
fp8bs_status fp8bs_quant_act_1x128(const void *x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t *q, int64_t ldq, float *s, int64_t lds,
                                   void *stream);

/*
 * Weight quantization with 128x128 blocks.
 * [p1] para 3: the max-abs is taken online for every 128x128 weight block.
 *   w  bf16 [N][ldw]            input, row n holds K values
 *   q  u8   [N][ldq]            E4M3 codes
 *   s  f32  [ceil(N/128)][lds]  s[(n/128)*lds + k/128]
 * N may be ragged: the last block row takes its max-abs over the rows
 * present.  N >= 0, K > 0, K % 128 == 0.
 */
fp8bs_status fp8bs_quant_w_128x128(const void *w, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t *q, int64_t ldq, float *s, int64_t lds,
                                   void *stream);

/*
 * A layer's activation and weight quantized in one launch: exactly
 * fp8bs_quant_act_1x128(x, M, K, ...) and fp8bs_quant_w_128x128(w, N, K,
 * ...) ([p1] para 3: 1x128 activation tiles, 128x128 weight blocks), with
 * the same codes and scales, run as one kernel so that the two streams
 * share one ramp-up and drain and the activation runs beside the weight
 * blocks.
 *   x  bf16 [M][ldx]   qx u8 [M][ldqx]   sx f32 [M][ldsx]          (K/128 per row)
 *   w  bf16 [N][ldw]   qw u8 [N][ldqw]   sw f32 [ceil(N/128)][ldsw] (K/128 per row)
 * M >= 0, N >= 0 (a zero side is skipped, both zero is a no-op), K > 0 and
 * K % 128 == 0.  Arguments of a non-empty side are checked as in the
 * single calls; the two sides must not overlap.
 */
fp8bs_status fp8bs_quant_act_w(const void *x, int64_t M, int64_t ldx, uint8_t *qx, int64_t ldqx,
                               float *sx, int64_t ldsx, const void *w, int64_t N, int64_t ldw,
                               uint8_t *qw, int64_t ldqw, float *sw, int64_t ldsw, int64_t K,
                               void *stream);

/*
 * Per-tensor scaling: one scale for a whole tensor, the common practice
 * [p3] para 4 describes (the tensor's max-abs mapped to the FP8 maximum)
 * and [p1] para 4 contrasts with the fine-grained tiles.  The comparison
 * path of the accuracy study; its codes feed fp8bs_gemm with the scale
 * broadcast into the scale arrays.
 *   x  bf16 [n] (contiguous)     q  u8 [n]     s  f32 [1]
 * s = fl32(amax / 448) over all n values, q[i] = nearest-even E4M3 of
 * x[i] / s, saturated (as for a tile of fp8bs_quant_act_1x128).  s is also
 * used as working memory during the call.  n >= 0 (0 is a no-op),
 * n % 128 == 0, else FP8BS_ERR_UNSUPPORTED_SHAPE; x and q 16-byte aligned.
 */
fp8bs_status fp8bs_quant_per_tensor(const void *x, int64_t n, uint8_t *q, float *s, void *stream);

/*
 * FP32 -> E4M3 codes, nearest-even with saturation: the last step of every
 * quantizer here ([p1] para 3: a tile, divided by its scaling factor, is
 * quantized to FP8), run with a unit scale by the same encoder.  For data
 * whose scale is already applied, and a direct check of the encoder on any
 * FP32 value.
 *   x  f32 [n] (contiguous)     q  u8 [n]
 * q[i] = the E4M3 code nearest to x[i], ties to the even code, |x[i]| > 448
 * (infinities included) saturated to +-448, the sign of zero kept.  NaN
 * inputs give an unspecified code.  n >= 0 (0 is a no-op); x and q 16-byte
 * aligned, else FP8BS_ERR_MISALIGNED.
 */
fp8bs_status fp8bs_cast_e4m3(const float *x, int64_t n, uint8_t *q, void *stream);

/*
 * The 12-bit E5M6 format for cached activations.  [p1] para 3: a custom
 * E5M6 format is used for some activations cached for the backward pass.
 * Layout (a reading; the pages give none): bit 11 sign, bits 10..6
 * exponent with bias 15, bits 5..0 mantissa, IEEE conventions (exponent 0:
 * subnormal mant * 2^-20; exponent 31: infinity or NaN); largest finite
 * value 65024.  A row of C values is packed into 1.5 C bytes, value i in
 * bits 12 i .. 12 i + 11, little-endian.
 * Encoding rounds each bf16 value to the nearest E5M6 value, ties to the
 * even mantissa, magnitudes from 65280 up to infinity (IEEE overflow).
 * Every E5M6 value is a bf16 value, so decoding is exact; in the backward
 * pass fp8bs_requant_T_128x1 takes the packed rows directly (FP8BS_SRC_E5M6),
 * with the result it gives for the decoded rows as FP8BS_SRC_BF16.
 *   x  bf16 [T][ldx]     y  u8 [T][ldy]  (ldy in bytes, >= 1.5 C)
 * T >= 0 (0 is a no-op), C > 0, C % 128 == 0, else
 * FP8BS_ERR_UNSUPPORTED_SHAPE; 16-byte alignment as for every byte buffer.
 */
fp8bs_status fp8bs_encode_e5m6(const void *x, int64_t T, int64_t C, int64_t ldx, uint8_t *y,
                               int64_t ldy, void *stream);
fp8bs_status fp8bs_decode_e5m6(const uint8_t *y, int64_t T, int64_t C, int64_t ldy, void *x,
                               int64_t ldx, void *stream);

/*
 * SwiGLU of the cached gate and up halves, quantized for the down-projection.
 * [p1] para 4 and [p4] para 3 cache the inputs of the SwiGLU operator and
 * recompute its output in the backward pass; [p1] para 3 quantizes a GEMM
 * input in 1x128 tiles along its K (here I); [p2] para 1 counts the HBM
 * round trip that a separate quantization costs.
 *   h = silu(g) * u = g * u / (1 + e^-g), computed in FP32 (within a few
 *   units in the last place of the exact value where it is normal)
 *   g, u  bf16 [T][ldg], [T][ldu]   the two halves (a [T][2I] up-projection
 *                                   output: u = g + I, ldu = ldg)
 *   q, s  u8 [T][ldq], f32 [T][lds] E4M3 codes and 1x128 scales of h,
 *                                   s = fl32(amax / 448), codes the
 *                                   nearest-even E4M3 of h / s (as
 *                                   fp8bs_quant_act_1x128 quantizes FP32
 *                                   values); both or neither
 *   h     bf16 [T][ldh] or NULL     h rounded to nearest-even BF16 (the
 *                                   backward pass's recompute)
 * At least one output.  T >= 0 (0 is a no-op), I > 0 and I % 128 == 0, else
 * FP8BS_ERR_INVALID_ARG / FP8BS_ERR_UNSUPPORTED_SHAPE; buffers and row
 * strides 16-byte aligned.  NaN and infinite inputs are outside the
 * contract.
 */
fp8bs_status fp8bs_swiglu_quant_1x128(const void *g, int64_t ldg, const void *u, int64_t ldu,
                                      int64_t T, int64_t I, uint8_t *q, int64_t ldq, float *s,
                                      int64_t lds, void *h, int64_t ldh, void *stream);

/*
 * Backward re-quantization of 1x128 tiles into 128x1 tiles, transposed.
 * [p1] para 3: in the backward pass the activation tiles are converted
 * from 1x128 to 128x1; [p1] para 4: activations are cached in FP8 for the
 * backward pass of the Linear operator.
 * Reading: v = fl32(dec(q_in[t][c]) * s_in[t][c/128]) (one FP32 multiply);
 * for src == FP8BS_SRC_BF16, v = x[t][c] and s_in is ignored (may be NULL);
 * for src == FP8BS_SRC_E5M6 ([p1] para 3: E5M6 for activations cached for
 * the backward pass), v = the E5M6 value packed at x[t][1.5 c] (ld_in in
 * bytes; decoding is exact, so the result is that of FP8BS_SRC_BF16 on the
 * decoded rows, without their round trip through HBM) and s_in is ignored.
 * Each run of 128 consecutive tokens t of one channel c is a tile; the
 * result is written channel-major so that T becomes the contiguous (K)
 * dimension of a following GEMM.
 *   in     u8 [T][ld_in] (codes), bf16 [T][ld_in], or u8 [T][ld_in] (E5M6, >= 1.5 C bytes)
 *   s_in   f32 [T][lds_in]            s_in[t*lds_in + c/128]
 *   q_out  u8  [C][ld_out]            q_out[c*ld_out + t]
 *   s_out  f32 [C][lds_out]           s_out[c*lds_out + t/128], ceil(T/128) per row
 * T may be ragged (the last token tile takes its max-abs over the tokens
 * present).  T >= 0, C > 0, C % 128 == 0; an input row must span fewer
 * than 2^25 bytes (ld_in) and lds_in < 2^22, else
 * FP8BS_ERR_UNSUPPORTED_SHAPE.
 */
fp8bs_status fp8bs_requant_T_128x1(fp8bs_requant_src src, const void *in, const float *s_in,
                                   int64_t T, int64_t C, int64_t ld_in, int64_t lds_in,
                                   uint8_t *q_out, int64_t ld_out, float *s_out, int64_t lds_out,
                                   void *stream);

/*
 * Transpose of 128x128-block-quantized weights, for the backward pass for
 * the input.  [p3] para 4: the backward pass is split into a part for the
 * input and a part for the weights; [p1] para 3: weights are quantized in
 * 128x128 blocks.  dX = dY W needs W as the B operand of fp8bs_gemm
 * (K-contiguous), i.e. as W^T.  A block's max-abs does not depend on its
 * orientation, so the quantized W^T is the transposed codes of W with the
 * transposed scale grid (the same bits fp8bs_quant_w_128x128 gives for the
 * bf16 W^T); nothing is re-quantized.
 *   q   u8  [N][ldq]    codes of W            s   f32 [N/128][lds]    s[(n/128)*lds + k/128]
 *   qt  u8  [K][ldqt]   qt[k*ldqt + n] = q[n*ldq + k]
 *   st  f32 [K/128][ldst]  st[(k/128)*ldst + n/128] = s[(n/128)*lds + k/128]
 * N >= 0 (0 is a no-op), K > 0; N % 128 == 0 and K % 128 == 0 (the
 * transposed weight is the K-contiguous operand of a GEMM with K' = N),
 * and a code row must span fewer than 2^25 bytes (ldq), else
 * FP8BS_ERR_UNSUPPORTED_SHAPE.  q and qt must not overlap.
 */
fp8bs_status fp8bs_transpose_w_128x128(const uint8_t *q, int64_t N, int64_t K, int64_t ldq,
                                       const float *s, int64_t lds, uint8_t *qt, int64_t ldqt,
                                       float *st, int64_t ldst, void *stream);

/*
 * Block-scaled FP8 GEMM, D = A * B^T, both operands K-contiguous.
 * [p1] para 2: per-group scales along K are multiplied in as part of
 * dequantization; [p1] para 3 and [p2] para 1: partial sums are promoted to
 * FP32 accumulation; [p4] para 4: FP8 inputs, BF16 or FP32 output.
 * Computed: D[m][n] = sum_g sa[m][g] * sb(n, g) * P_g[m][n] with
 * P_g = sum over the 128 k of group g of dec(a[m][k]) * dec(b[n][k]);
 * each P_g is formed in FP32 and added into an FP32 accumulator once per
 * 128-wide K group, then rounded once to the output type (BF16: nearest-even).
 *   a   u8  [M][lda]      sa f32 [M][ldsa]       sa[m*ldsa + k/128]
 *   b   u8  [N][ldb]      sb f32, layout by bmode (see fp8bs_bscale)
 *   d   bf16 or f32 [M][ldd]
 * M, N >= 0 (either 0 is a no-op); K > 0, K % 128 == 0.  M and N may be
 * ragged.  lda, ldb < 2^24 and ldsa, ldsb < 2^22, else
 * FP8BS_ERR_UNSUPPORTED_SHAPE.
 */
fp8bs_status fp8bs_gemm(const uint8_t *a, const float *sa, int64_t lda, int64_t ldsa,
                        const uint8_t *b, const float *sb, int64_t ldb, int64_t ldsb,
                        fp8bs_bscale bmode, void *d, int64_t ldd, fp8bs_out_dtype dt,
                        int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Block-scaled FP8 GEMM whose result leaves already quantized for the next
 * layer: the quantization of the output activations is fused into the
 * GEMM's epilogue, so the output crosses HBM once, as E4M3 codes, instead
 * of being written in BF16 and read back by fp8bs_quant_act_1x128 ([p2]
 * para 1 describes that round trip as the cost of separate quantization).
 * D is computed as by fp8bs_gemm (FP32 per-group promotion); each 1x128
 * tile of D along N (row m, columns 128j .. 128j+127) is then quantized
 * from its FP32 values as fp8bs_quant_act_1x128 quantizes a tile:
 * s = fl32(amax / 448), q = nearest-even E4M3 of d / s, saturated.
 *   a, sa, b, sb, bmode   as for fp8bs_gemm
 *   q  u8  [M][ldq]       E4M3 codes of D
 *   s  f32 [M][lds]       s[m*lds + n/128]
 * M >= 0, N >= 0 (either 0 is a no-op), K > 0; K % 128 == 0 and
 * N % 128 == 0, else FP8BS_ERR_UNSUPPORTED_SHAPE (also for the stride
 * limits of fp8bs_gemm).
 */
fp8bs_status fp8bs_gemm_quant_1x128(const uint8_t *a, const float *sa, int64_t lda, int64_t ldsa,
                                    const uint8_t *b, const float *sb, int64_t ldb, int64_t ldsb,
                                    fp8bs_bscale bmode, uint8_t *q, int64_t ldq, float *s,
                                    int64_t lds, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Block-scaled FP8 GEMM whose A operand is given in BF16 and quantized in
 * 1x128 tiles inside the GEMM, so the FP8 activation never crosses HBM
 * ([p2] para 1 describes the HBM round trip of separate quantization: BF16
 * read, FP8 written back, read again for the MMA).  Each tile of A is
 * quantized exactly as fp8bs_quant_act_1x128 quantizes it ([p1] para 3)
 * and D is then computed as by fp8bs_gemm on those codes with 128x128 B
 * scales (bit for bit the same D).  Each 64-row tile of A is quantized once
 * per 256-column tile of B, so the form is meant for small N.
 *   x   bf16 [M][ldx]          A
 *   qx  u8   [M][ldqx] or NULL the E4M3 codes of A are also stored (the FP8
 *   sx  f32  [M][ldsx] or NULL activation cache for the backward pass);
 *                              both given or both NULL
 *   b, sb, ldb, ldsb           as for fp8bs_gemm with FP8BS_BSCALE_BLOCK_128x128
 *   d   bf16 or f32 [M][ldd]
 * M, N >= 0 (either 0 is a no-op), K > 0, K % 128 == 0; ldx < 2^23,
 * ldb < 2^24, ldsb < 2^22, else FP8BS_ERR_UNSUPPORTED_SHAPE.
 */
fp8bs_status fp8bs_gemm_bf16a(const void *x, int64_t ldx, uint8_t *qx, int64_t ldqx, float *sx,
                              int64_t ldsx, const uint8_t *b, const float *sb, int64_t ldb,
                              int64_t ldsb, void *d, int64_t ldd, fp8bs_out_dtype dt, int64_t M,
                              int64_t N, int64_t K, void *stream);

/*
 * Grouped block-scaled GEMM for the experts one GPU holds, with ragged
 * token counts (the per-expert FP8 GEMMs of the MoE layers; [p2] para 2).
 * Rows offsets[e] .. offsets[e+1]-1 of A are multiplied by expert e:
 *   D[m][n] = sum_g sa[m][g] * sb[e][n/128][g] * P_g(m, n; b[e])
 *   a        u8  [M_total][K] (dense rows)   sa f32 [M_total][ldsa]
 *   b        u8  [E][N][K] (dense)            sb f32 [E][ceil(N/128)][K/128] (dense)
 *   offsets  i32 [E+1] in DEVICE memory, offsets[0] = 0,
 *            non-decreasing, offsets[E] = M_total (not checked: a
 *            violation gives unspecified rows but no out-of-bounds access)
 *   d        bf16 or f32 [M_total][N] (dense)
 * M_total sizes the launch only; no host synchronization.
 * E >= 1, M_total >= 0, N > 0, K > 0, K % 128 == 0; K < 2^24 and
 * ldsa < 2^22, else FP8BS_ERR_UNSUPPORTED_SHAPE.
 */
fp8bs_status fp8bs_grouped_gemm(const uint8_t *a, const float *sa, int64_t ldsa,
                                const uint8_t *b, const float *sb,
                                const int32_t *offsets, int32_t E, int64_t M_total,
                                void *d, fp8bs_out_dtype dt, int64_t N, int64_t K,
                                void *stream);

/* Human-readable name of a status code (static storage). */
const char *fp8bs_status_string(fp8bs_status st);

/* Version of the library as major*10000 + minor*100 + patch. */
int fp8bs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
