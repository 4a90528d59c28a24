/*
 * fp8bs_oracle.c -- CPU oracle for fine-grained FP8 quantization and the
 * block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant with the GPU library, and the GPU
 * library never calls it.
 *
 * Sources.  The method is taken from the DeepSeek-V3 report excerpts on five
 * web pages, cited here as
 *   [p1] xn--9g3bo1gtkw0l8ubf92bgle.kr board post wr_id=32373
 *   [p2] why-be.why-be.co.kr board post wr_id=73620
 *   [p4] bestpmk.kr board post wr_id=299512
 * with a paragraph number (1-based, counted on that page).  The pages fix the
 * tile geometry and the dequantization relation; the number format (OCP
 * E4M3FN, largest finite value 448), the scale formula amax/448, rounding to
 * nearest-even with saturation, FP32 scales and the promotion interval of
 * 128 along K are the readings this project adopts where the pages only say
 * "FP8" (see the readings list of the design notes).
 *
 * Arithmetic rules.
 *   - Scales are IEEE binary32 and are computed in binary32, because the
 *     scale is a stored FP32 quantity.  Compile without fast-math and with
 *     -ffp-contract=off so that every float operation is a single correctly
 *     rounded IEEE operation with subnormals.
 *   - Quotients x/s are taken in binary64 and rounded once to E4M3.  Double
 *     rounding 53 -> 4 significant bits of a quotient is innocuous.
 *   - GEMM results are accumulated in binary64 and rounded once to the
 *     output type.
 * Parallel loops (OpenMP) only split independent output rows; they never
 * change the order of any sum.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the parallel loops use (1 without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* E4M3FN codec (OCP 8-bit floating point, E4M3 variant).               */
/* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.         */
/* exponent 0: subnormal, value mant * 2^-9.                            */
/* exponent 1..15: (8 + mant) * 2^(exp - 10); exp 15 with mant 7 = NaN. */
/* No infinities.                                                        */
/* ------------------------------------------------------------------ */

double orc_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp((double)(8 + m), e - 10);
    return sign ? -mag : mag;
}

/* Magnitude table of the 127 non-negative finite codes 0x00..0x7E.  The
 * codes are ordered by value, so index == code.  Filled once when the
 * library is loaded, before any (parallel) caller can use it. */
static double g_mag[127];

__attribute__((constructor)) static void build_mag_table(void)
{
    for (int c = 0; c < 127; ++c)
        g_mag[c] = orc_e4m3_value((uint8_t)c);
}

/* Round a finite binary64 value to the nearest E4M3 code, ties to the code
 * with an even mantissa, magnitudes beyond 448 saturate to 448.  Brute
 * force: binary search for the bracketing pair of representable magnitudes,
 * then compare against their exact midpoint. */
uint8_t orc_e4m3_encode(double y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    if (a >= g_mag[126])
        return sign | 126;
    int lo = 0, hi = 126; /* invariant: g_mag[lo] <= a < g_mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_mag[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    if (g_mag[lo] == a)
        return sign | (uint8_t)lo;
    /* midpoint of two E4M3 magnitudes is exact in binary64 */
    double midpoint = 0.5 * (g_mag[lo] + g_mag[hi]);
    int pick;
    if (a < midpoint)
        pick = lo;
    else if (a > midpoint)
        pick = hi;
    else
        pick = (lo % 2 == 0) ? lo : hi; /* even mantissa == even code */
    return sign | (uint8_t)pick;
}

/* ------------------------------------------------------------------ */
/* BF16 helpers                                                          */
/* ------------------------------------------------------------------ */

double orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a finite binary64 value to bfloat16, nearest-even, straight from
 * binary64 (one rounding).  Overflow past the largest finite bf16 goes to
 * infinity as IEEE rounding does. */
uint16_t orc_bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) */
    int exp_unb = e - 1;     /* a in [2^exp_unb, 2^(exp_unb+1)) */
    if (exp_unb < -126)
        exp_unb = -126;      /* subnormal bf16: fixed quantum 2^-133 */
    double quantum = ldexp(1.0, exp_unb - 7);
    double k = a / quantum;  /* exact: power-of-two scaling */
    double fl = floor(k);
    double frac = k - fl;    /* exact */
    double r;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else
        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double rv = r * quantum; /* exact */
    float f = (float)rv;     /* rv has <= 8 significant bits: exact, or inf */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Quantization of one group of values to E4M3 with one FP32 scale.      */
/* [p1] para 3: the max absolute value is found online for each tile or   */
/* block, a scaling factor is derived from it, and the values are         */
/* quantized to FP8.  Reading adopted: s = fl32(amax / 448), code =       */
/* RNE_sat(x / s); an all-zero group gets s = 0 and signed-zero codes.    */
/* ------------------------------------------------------------------ */

static float scale_from_amax(float amax)
{
    volatile float d = 448.0f; /* keep it a real IEEE binary32 division */
    return amax / d;
}

static uint8_t quantize_one(float x, float s)
{
    if (s == 0.0f)
        return signbit(x) ? 0x80 : 0x00;
    return orc_e4m3_encode((double)x / (double)s);
}

/* Activation quantization, 1x128 tiles along K.
 * x: bf16 [M][K] row-major (ld = K); q: [M][K]; s: [M][K/128].
 * K must be a multiple of 128. */
void orc_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K,
                         uint8_t *q, float *s)
{
    int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < G; ++g) {
            float amax = 0.0f;
            for (int64_t k = g * 128; k < g * 128 + 128; ++k) {
                float v = fabsf((float)orc_bf16_value(x[m * K + k]));
                if (v > amax)
                    amax = v;
            }
            float sc = scale_from_amax(amax);
            s[m * G + g] = sc;
            for (int64_t k = g * 128; k < g * 128 + 128; ++k)
                q[m * K + k] = quantize_one((float)orc_bf16_value(x[m * K + k]), sc);
        }
    }
}

/* Activation quantization of an FP32 input (same tiles).  Used only to
 * state the backward re-quantization as a composition in the tests. */
void orc_quant_act_1x128_f32(const float *x, int64_t M, int64_t K,
                             uint8_t *q, float *s)
{
    int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < G; ++g) {
            float amax = 0.0f;
            for (int64_t k = g * 128; k < g * 128 + 128; ++k) {
                float v = fabsf(x[m * K + k]);
                if (v > amax)
                    amax = v;
            }
            float sc = scale_from_amax(amax);
            s[m * G + g] = sc;
            for (int64_t k = g * 128; k < g * 128 + 128; ++k)
                q[m * K + k] = quantize_one(x[m * K + k], sc);
        }
    }
}

/* SwiGLU of the cached gate and up halves, quantized for the
 * down-projection.  [p1] para 4 and [p4] para 3 cache the inputs of the
 * SwiGLU operator (recomputing its output in the backward pass); [p1]
 * para 3 quantizes the input of a GEMM in 1x128 tiles along its K.
 * Reading taken: h = silu(g) * u with silu(g) = g / (1 + e^-g), evaluated
 * in binary64 (libm exp) and rounded once to binary32; the binary32 rows
 * are then quantized exactly as orc_quant_act_1x128_f32 quantizes them.
 * g, u: bf16 [T][I]; q: [T][I]; s: [T][I/128]; h32: [T][I] (the rounded
 * h, for the tests); h16: [T][I] bf16 bits of h rounded once from
 * binary64, or NULL. */
static double silu_times(double g, double u)
{
    return g / (1.0 + exp(-g)) * u;
}

void orc_swiglu_quant_1x128(const uint16_t *g, const uint16_t *u, int64_t T,
                            int64_t I, uint8_t *q, float *s, float *h32,
                            uint16_t *h16)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < I; ++i) {
            double h = silu_times(orc_bf16_value(g[t * I + i]),
                                  orc_bf16_value(u[t * I + i]));
            h32[t * I + i] = (float)h;
            if (h16)
                h16[t * I + i] = orc_bf16_round(h);
        }
    }
    orc_quant_act_1x128_f32(h32, T, I, q, s);
}

/* Weight quantization, 128x128 blocks.
 * w: bf16 [N][K] (ld = K); q: [N][K]; s: [ceil(N/128)][K/128].
 * A partial last block row takes its amax over the rows present. */
void orc_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K,
                         uint8_t *q, float *s)
{
    int64_t G = K / 128;
    int64_t NB = (N + 127) / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t nb = 0; nb < NB; ++nb) {
        for (int64_t g = 0; g < G; ++g) {
            int64_t n_end = (nb + 1) * 128 < N ? (nb + 1) * 128 : N;
            float amax = 0.0f;
            for (int64_t n = nb * 128; n < n_end; ++n)
                for (int64_t k = g * 128; k < g * 128 + 128; ++k) {
                    float v = fabsf((float)orc_bf16_value(w[n * K + k]));
                    if (v > amax)
                        amax = v;
                }
            float sc = scale_from_amax(amax);
            s[nb * G + g] = sc;
            for (int64_t n = nb * 128; n < n_end; ++n)
                for (int64_t k = g * 128; k < g * 128 + 128; ++k)
                    q[n * K + k] = quantize_one((float)orc_bf16_value(w[n * K + k]), sc);
        }
    }
}

/* Backward re-quantization, 1x128 -> 128x1, written transposed.
 * [p1] para 3: in the backward pass the 1x128 activation tiles are turned
 * into 128x1 tiles.  Reading adopted: each value is first dequantized in
 * FP32, v = fl32(dec(q) * s1), then every run of 128 consecutive tokens of
 * one channel is quantized as a tile (amax, s2 = amax/448, RNE_sat(v/s2)).
 * src == 0: in = E4M3 codes [T][C] with s_in [T][C/128].
 * src == 1: in = bf16 [T][C] (a fresh gradient); s_in unused; v = x.
 * out: q_out [C][T]; s_out [C][ceil(T/128)].  C % 128 == 0. */
void orc_requant_T_128x1(int src, const void *in, const float *s_in,
                         int64_t T, int64_t C, uint8_t *q_out, float *s_out)
{
    int64_t GC = C / 128;
    int64_t GT = (T + 127) / 128;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        for (int64_t tg = 0; tg < GT; ++tg) {
            int64_t t_end = (tg + 1) * 128 < T ? (tg + 1) * 128 : T;
            float v[128];
            float amax = 0.0f;
            for (int64_t t = tg * 128; t < t_end; ++t) {
                float val;
                if (src == 0) {
                    const uint8_t *qi = (const uint8_t *)in;
                    float dq = (float)orc_e4m3_value(qi[t * C + c]);
                    val = dq * s_in[t * GC + c / 128]; /* one FP32 multiply */
                } else {
                    const uint16_t *xi = (const uint16_t *)in;
                    val = (float)orc_bf16_value(xi[t * C + c]);
                }
                v[t - tg * 128] = val;
                if (fabsf(val) > amax)
                    amax = fabsf(val);
            }
            float sc = scale_from_amax(amax);
            s_out[c * GT + tg] = sc;
            for (int64_t t = tg * 128; t < t_end; ++t)
                q_out[c * T + t] = quantize_one(v[t - tg * 128], sc);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Block-scaled GEMM, D = A * B^T.                                        */
/* [p1] para 2: per-group scaling factors along K are multiplied in as    */
/* part of dequantization.  [p4] para 4: FP8 inputs, BF16 or FP32 output. */
/* Definition implemented: D[m][n] = sum_k (dec(qa[m][k]) * sa[m][k/128]) */
/*                                        * (dec(qb[n][k]) * sb(n, k/128)) */
/* in binary64, k ascending, then one rounding by the caller.             */
/* bmode 0: sb is [ceil(N/128)][K/128] (128x128 weight blocks).           */
/* bmode 1: sb is [N][K/128] (1x128 tiles, the wgrad operand).            */
/* ------------------------------------------------------------------ */

static double b_scale(const float *sb, int bmode, int64_t n, int64_t g, int64_t G)
{
    if (bmode == 0)
        return (double)sb[(n / 128) * G + g];
    return (double)sb[n * G + g];
}

/* Dot product of one output entry. */
static double gemm_entry(const uint8_t *a, const float *sa,
                         const uint8_t *b, const float *sb, int bmode,
                         int64_t m, int64_t n, int64_t K)
{
    int64_t G = K / 128;
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double av = orc_e4m3_value(a[m * K + k]) * (double)sa[m * G + k / 128];
        double bv = orc_e4m3_value(b[n * K + k]) * b_scale(sb, bmode, n, k / 128, G);
        acc += av * bv;
    }
    return acc;
}

/* Full GEMM: d [M][N] binary64.  a [M][K], sa [M][K/128], b [N][K]. */
void orc_gemm(const uint8_t *a, const float *sa, const uint8_t *b,
              const float *sb, int bmode, int64_t M, int64_t N, int64_t K,
              double *d)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            d[m * N + n] = gemm_entry(a, sa, b, sb, bmode, m, n, K);
}

/* Selected entries only: d[i] = D[mi[i]][ni[i]]. */
void orc_gemm_entries(const uint8_t *a, const float *sa, const uint8_t *b,
                      const float *sb, int bmode, int64_t K,
                      const int64_t *mi, const int64_t *ni, int64_t count,
                      double *d)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i)
        d[i] = gemm_entry(a, sa, b, sb, bmode, mi[i], ni[i], K);
}

/* Grouped GEMM over experts.  Rows offsets[e] .. offsets[e+1]-1 of A use
 * expert e's weights b[e] ([N][K]) and block scales sb[e]
 * ([ceil(N/128)][K/128]).  d [offsets[E]][N] binary64. */
void orc_grouped_gemm(const uint8_t *a, const float *sa, const uint8_t *b,
                      const float *sb, const int32_t *offsets, int32_t E,
                      int64_t N, int64_t K, double *d)
{
    int64_t G = K / 128;
    int64_t NB = (N + 127) / 128;
    for (int32_t e = 0; e < E; ++e) {
        const uint8_t *be = b + (int64_t)e * N * K;
        const float *sbe = sb + (int64_t)e * NB * G;
        int64_t r0 = offsets[e], r1 = offsets[e + 1];
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t m = r0; m < r1; ++m)
            for (int64_t n = 0; n < N; ++n)
                d[m * N + n] = gemm_entry(a, sa, be, sbe, 0, m, n, K);
    }
}

/* Selected entries of the grouped GEMM; the expert of row mi[i] is found
 * from the offsets. */
void orc_grouped_gemm_entries(const uint8_t *a, const float *sa,
                              const uint8_t *b, const float *sb,
                              const int32_t *offsets, int32_t E, int64_t N,
                              int64_t K, const int64_t *mi, const int64_t *ni,
                              int64_t count, double *d)
{
    int64_t G = K / 128;
    int64_t NB = (N + 127) / 128;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int32_t e = 0;
        while (e < E && !(mi[i] >= offsets[e] && mi[i] < offsets[e + 1]))
            ++e;
        if (e == E) {
            d[i] = NAN;
            continue;
        }
        d[i] = gemm_entry(a, sa, b + (int64_t)e * N * K,
                          sb + (int64_t)e * NB * G, 0, mi[i], ni[i], K);
    }
}

/* Round an array of binary64 results to bf16 (one rounding each). */
void orc_round_to_bf16(const double *v, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_round(v[i]);
}

/* ------------------------------------------------------------------ */
/* Accuracy-probe references (context for the K = 4096 probe).          */
/* ------------------------------------------------------------------ */

/* Unquantized GEMM of the bf16 inputs in binary64: d = X * W^T. */
void orc_gemm_bf16_f64(const uint16_t *x, const uint16_t *w, int64_t M,
                       int64_t N, int64_t K, double *d)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += orc_bf16_value(x[m * K + k]) * orc_bf16_value(w[n * K + k]);
            d[m * N + n] = acc;
        }
}

/* BF16 GEMM as a plain FP32-accumulating kernel would run it: products of
 * the bf16 inputs summed in binary32, k ascending; the caller rounds the
 * binary32 result to bf16. */
void orc_gemm_bf16_f32acc(const uint16_t *x, const uint16_t *w, int64_t M,
                          int64_t N, int64_t K, float *d)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float p = (float)orc_bf16_value(x[m * K + k]) *
                          (float)orc_bf16_value(w[n * K + k]); /* exact */
                acc += p;
            }
            d[m * N + n] = acc;
        }
}

/* Limited-precision accumulation without promotion, after the H800
 * description ([p1] para 3: about 14 retained bits; [p2] para 3: only the
 * top 14 bits of each mantissa product survive, after a sign-filling right
 * shift, lower bits are truncated).  Reading adopted (context only; pinned
 * by hand-worked cases in tests/golden/unpromoted_hand.json): per-tensor
 * scales sa_t, sb_t; the K products of the raw
 * E4M3 codes are taken in chunks of `chunk` products; for each chunk, the
 * running accumulator and the chunk's products are aligned to the largest
 * exponent among them, each is truncated toward minus infinity to `bits`
 * bits below that exponent's leading bit, and the truncated values are
 * summed exactly; the result is carried to the next chunk and never
 * promoted to a wider accumulator.  d = sa_t * sb_t * acc. */
static double trunc_to(double v, int lead_exp, int bits)
{
    /* keep multiples of 2^(lead_exp - bits + 1), rounding toward -inf
     * (an arithmetic right shift of a two's-complement value) */
    double q = ldexp(1.0, lead_exp - bits + 1);
    return floor(v / q) * q;
}

void orc_gemm_unpromoted(const uint8_t *a, float sa_t, const uint8_t *b,
                         float sb_t, int64_t M, int64_t N, int64_t K,
                         int chunk, int bits, double *d)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k0 = 0; k0 < K; k0 += chunk) {
                int64_t k1 = k0 + chunk < K ? k0 + chunk : K;
                double maxabs = fabs(acc);
                for (int64_t k = k0; k < k1; ++k) {
                    double p = orc_e4m3_value(a[m * K + k]) * orc_e4m3_value(b[n * K + k]);
                    if (fabs(p) > maxabs)
                        maxabs = fabs(p);
                }
                if (maxabs == 0.0)
                    continue;
                int e;
                frexp(maxabs, &e);
                int lead = e - 1;
                double sum = trunc_to(acc, lead, bits);
                for (int64_t k = k0; k < k1; ++k) {
                    double p = orc_e4m3_value(a[m * K + k]) * orc_e4m3_value(b[n * K + k]);
                    sum += trunc_to(p, lead, bits);
                }
                acc = sum;
            }
            d[m * N + n] = acc * (double)sa_t * (double)sb_t;
        }
}

/* Per-tensor quantization (the standard practice the pages contrast with,
 * [p1] para 4): one scale for the whole tensor, s = fl32(amax/448). */
void orc_quant_per_tensor(const uint16_t *x, int64_t n, uint8_t *q, float *s)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf((float)orc_bf16_value(x[i]));
        if (v > amax)
            amax = v;
    }
    float sc = scale_from_amax(amax);
    *s = sc;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        q[i] = quantize_one((float)orc_bf16_value(x[i]), sc);
}

/* ------------------------------------------------------------------ */
/* E5M6 cached-activation format ([p1] para 3 names a custom E5M6 format */
/* for some cached activations; the layout below is the reading taken): */
/* 12 bits, bit 11 sign, bits 10..6 exponent (bias 15), bits 5..0       */
/* mantissa, IEEE conventions: exponent 0 subnormal (mant * 2^-20),      */
/* exponent 31 infinity (mant 0) or NaN.                                 */
/* ------------------------------------------------------------------ */

double orc_e5m6_value(uint16_t code)
{
    int sign = (code >> 11) & 1;
    int e = (code >> 6) & 31;
    int m = code & 63;
    double mag;
    if (e == 31)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m, -20);
    else
        mag = ldexp((double)(64 + m), e - 21);
    return sign ? -mag : mag;
}

/* Nearest E5M6 code of a binary64 value, ties to the even mantissa; values
 * at or beyond the midpoint between the largest finite value and 2^16 round
 * to infinity (IEEE round-to-nearest overflow).  Brute force over the
 * ordered table of the 1984 non-negative finite magnitudes (codes 0..0x7BF
 * are ordered by value). */
static double g_m6[1984];

__attribute__((constructor)) static void build_m6_table(void)
{
    for (int c = 0; c < 1984; ++c)
        g_m6[c] = orc_e5m6_value((uint16_t)c);
}

uint16_t orc_e5m6_encode(double y)
{
    uint16_t sign = signbit(y) ? 0x800 : 0;
    double a = fabs(y);
    double top = g_m6[1983];
    double over = top + 0.5 * (65536.0 - top); /* midpoint to 2^16 */
    if (a >= over)
        return sign | 0x7C0;                    /* infinity (ties go to even 2^16) */
    if (a >= top)
        return sign | 1983;
    int lo = 0, hi = 1983;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_m6[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    if (g_m6[lo] == a)
        return sign | (uint16_t)lo;
    double midpoint = 0.5 * (g_m6[lo] + g_m6[hi]);
    int pick;
    if (a < midpoint)
        pick = lo;
    else if (a > midpoint)
        pick = hi;
    else
        pick = (lo % 2 == 0) ? lo : hi;
    return sign | (uint16_t)pick;
}

/* bf16 [T][C] -> packed E5M6 rows (value i of a row in bits 12 i .. 12 i + 11,
 * little-endian), C even. */
void orc_encode_e5m6(const uint16_t *x, int64_t T, int64_t C, uint8_t *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < C; i += 2) {
            uint16_t c0 = orc_e5m6_encode(orc_bf16_value(x[t * C + i]));
            uint16_t c1 = orc_e5m6_encode(orc_bf16_value(x[t * C + i + 1]));
            uint8_t *p = y + t * (C / 2 * 3) + i / 2 * 3;
            p[0] = (uint8_t)(c0 & 0xFF);
            p[1] = (uint8_t)((c0 >> 8) | ((c1 & 0xF) << 4));
            p[2] = (uint8_t)(c1 >> 4);
        }
}

/* packed E5M6 rows -> bf16 (every E5M6 value is a bf16 value) */
void orc_decode_e5m6(const uint8_t *y, int64_t T, int64_t C, uint16_t *x)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < C; i += 2) {
            const uint8_t *p = y + t * (C / 2 * 3) + i / 2 * 3;
            uint16_t c0 = (uint16_t)(p[0] | ((p[1] & 0xF) << 8));
            uint16_t c1 = (uint16_t)((p[1] >> 4) | (p[2] << 4));
            x[t * C + i] = orc_bf16_round(orc_e5m6_value(c0));
            x[t * C + i + 1] = orc_bf16_round(orc_e5m6_value(c1));
        }
}
