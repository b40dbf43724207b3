/*
 * ConvRot W8A8 / W4A8 linear -- CPU ORACLE (test infrastructure only).
 *
 * This file is the plain, slow, obviously-correct definition of what the
 * ConvRot quantized linear computes.  It exists so that tests, the smoke check
 * and the benchmark's CPU-baseline leg can check the HIP library against it.
 * It is NOT part of the product path: nothing in the library links, loads or
 * calls it, and it shares no code, header, table or constant with the GPU
 * kernels.
 *
 * Sources (web pages on ConvRot int8/int4 checkpoints):
 *  [P1] "MOSS-Image Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", file table,
 *       rows "Quantized" and "Matmul".
 *  [P2] "qwen3.5_4b_int8_convrot", sections "Why ConvRot" and
 *       "Quantization Recipe" (--scaling_mode row --simple, group size 256).
 *  [P3] "qwen3vl_8b_int8_convrot", section "Layer and group selection".
 *  [P4] "craftingmod/Qwen3-VL-8B-Heretic-INT8", section "Quantization metadata"
 *       (convrot, convrot_groupsize 256, per_row, orig_dtype bfloat16).
 *  [P5] "MossInt4", section "Format" (signed 4-bit codes two per byte, one F32
 *       scale per row chosen by a clip search, 8-bit activations).
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *  - Hadamard: Sylvester construction in natural order,
 *    H[i][j] = (-1)^popcount(i & j) / sqrt(g); rotation is x' = x * H applied
 *    to each contiguous group of g columns along K.  g = 1 means no rotation.
 *  - Precision: the rotation is computed here in fp64 by an explicit dense
 *    matrix product (not a fast transform) and is never rounded to a narrower
 *    type.  The absmax is taken over those fp64 values; the scale alone is
 *    rounded to fp32 (the pages store one fp32 scale per row); each code is
 *    decided on the fp64 quotient value / (double)scale.  This is the plain
 *    definition; a kernel that rotates and divides in fp32 can land on the
 *    other side of a rounding boundary, by one code, on rare elements.
 *  - scale = (float)(absmax / 127); code = round_half_away_from_zero(value /
 *    scale) clamped to [-127, 127]; an all-zero row gets scale 0 and codes 0.
 *  - GEMM: naive triple loop, exact integer accumulation.
 *  - Epilogue: y = bf16_rne(((float)acc * s_x[m]) * s_w[n]) in fp32.
 *  - int4: codes in [-7, 7]; clip factor c from 1.00 down to 0.50 in steps of
 *    0.01; scale = (float)(c * absmax / 7) with the fp64 absmax; codes decided
 *    on the fp64 quotient as for int8; the c with the smallest sum of squared
 *    reconstruction error (fp64, against the fp64 rotated row) wins (ties to
 *    the larger c); byte j of a row holds column 2j in its low nibble and
 *    column 2j+1 in its high nibble.
 *  - Weight-only (dequant) path ([P1] row "Matmul", [P2]): W^ = (wq * s_w)
 *    * H, with the integer +-1 transform of the codes taken exactly and the
 *    1/sqrt(g) applied once (so only that irrational constant rounds), a zero
 *    result +0, rounded to fp32 and then to bf16; then a bf16 matmul whose
 *    sum is taken in fp64 and rounded to fp32 and then to bf16.
 *  - RMSNorm before the linear ([P1] rows "Changed" and "How it was made":
 *    SmoothQuant scales folded into the norm weight as (1 + w) / s - 1): the
 *    norm multiplies by (1 + w); mean square over the whole row, eps inside
 *    the square root; fp32 arithmetic except the fp64 sum of squares; the
 *    output is rounded to bf16 (the activation dtype) before it is rotated.
 *
 * Build: gcc -std=c11 -O2 -fopenmp -ffp-contract=off -shared -fPIC.
 * OpenMP is used only to run independent rows in parallel; every row is
 * computed by the same sequential loop.
 *
 * parity: every function below is pinned by the CPU tests (closed forms,
 * library routines, brute force on tiny inputs); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_OVERFLOW 2

/* ---------------------------------------------------------------- helpers */

/* bf16 bit pattern -> fp64, exact (bf16 is the top half of an fp32). */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even.  The 16 dropped
 * mantissa bits are compared with one half of the kept unit in the last
 * place; NaN stays a quiet NaN. */
static uint16_t float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* Round half away from zero (C's round is exactly this). */
static double round_half_away(double v) { return round(v); }

static int is_pow2(int64_t g) { return g > 0 && (g & (g - 1)) == 0; }

/* ---------------------------------------------------------- the Hadamard */

/* H[i*g + j] = (-1)^popcount(i & j) / sqrt(g), Sylvester order. */
void oracle_hadamard(int g, double *H) {
    double norm = 1.0 / sqrt((double)g);
    for (int i = 0; i < g; ++i)
        for (int j = 0; j < g; ++j)
            H[(int64_t)i * g + j] = (__builtin_popcount((unsigned)(i & j)) & 1) ? -norm : norm;
}

/* Rotate one row of K values in fp64: for every group of g contiguous
 * columns, out[j] = sum_i in[i] * H[i][j] (dense product, [P1] "Quantized"
 * and "Matmul" rows: one rotation serves the weight rows and the
 * activations). */
static void rotate_row_f64(const double *in, int64_t K, int g, const double *H, double *out) {
    for (int64_t base = 0; base < K; base += g) {
        for (int j = 0; j < g; ++j) {
            double acc = 0.0;
            for (int i = 0; i < g; ++i)
                acc += in[base + i] * H[(int64_t)i * g + j];
            out[base + j] = acc;
        }
    }
}

/* rows x K fp64 -> rotated fp64 (exposed for the identity tests). */
int oracle_rotate_rows(const double *x, int64_t rows, int64_t K, int g, double *out) {
    if (!x || !out || rows < 0 || K <= 0 || !is_pow2(g) || K % g) return ORACLE_ERR_ARG;
    double *H = (double *)malloc(sizeof(double) * (size_t)g * (size_t)g);
    if (!H) return ORACLE_ERR_ARG;
    oracle_hadamard(g, H);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        rotate_row_f64(x + r * K, K, g, H, out + r * K);
    free(H);
    return ORACLE_OK;
}

/* ------------------------------------------------- int8 row quantization */

/* Quantize one rotated row (fp64 values) with a symmetric int8 grid:
 * scale = (float)(absmax/127), code = round_half_away(v / scale) on the fp64
 * quotient.  ([P1] "Quantized": int8 with one fp32 scale per output row;
 * "Matmul": activations get one int8 scale per token; [P2] "Quantization
 * Recipe": --scaling_mode row --simple, i.e. plain rounding.) */
static void quantize_row_i8(const double *v, int64_t K, int8_t *q, float *scale) {
    double amax = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = fabs(v[k]);
        if (a > amax) amax = a;
    }
    float s = (float)(amax / 127.0);
    *scale = s;
    for (int64_t k = 0; k < K; ++k) {
        if (s == 0.0f) { q[k] = 0; continue; }
        double r = round_half_away(v[k] / (double)s);
        if (r > 127.0) r = 127.0;
        if (r < -127.0) r = -127.0;
        q[k] = (int8_t)r;
    }
}

/* Weight preparation, int8: W fp32 [N,K] -> wq int8 [N,K], scale fp32 [N]. */
int oracle_quantize_weight_i8(const float *w, int64_t N, int64_t K, int g, int8_t *wq, float *scale) {
    if (!w || !wq || !scale || N < 0 || K <= 0 || !is_pow2(g) || K % g) return ORACLE_ERR_ARG;
    double *H = (double *)malloc(sizeof(double) * (size_t)g * (size_t)g);
    if (!H) return ORACLE_ERR_ARG;
    oracle_hadamard(g, H);
#pragma omp parallel
    {
        double *in = (double *)malloc(sizeof(double) * (size_t)K);
        double *rot = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) in[k] = (double)w[n * K + k];
            rotate_row_f64(in, K, g, H, rot);
            quantize_row_i8(rot, K, wq + n * K, scale + n);
        }
        free(in); free(rot);
    }
    free(H);
    return ORACLE_OK;
}

/* Activation rotate + per-token quantization: x bf16 [M,K] -> xq int8 [M,K],
 * x_scale fp32 [M] ([P1] "Matmul" row). */
int oracle_rotate_quant(const uint16_t *x, int64_t M, int64_t K, int g, int8_t *xq, float *x_scale) {
    if (!x || !xq || !x_scale || M < 0 || K <= 0 || !is_pow2(g) || K % g) return ORACLE_ERR_ARG;
    double *H = (double *)malloc(sizeof(double) * (size_t)g * (size_t)g);
    if (!H) return ORACLE_ERR_ARG;
    oracle_hadamard(g, H);
#pragma omp parallel
    {
        double *in = (double *)malloc(sizeof(double) * (size_t)K);
        double *rot = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t k = 0; k < K; ++k) in[k] = bf16_bits_to_double(x[m * K + k]);
            rotate_row_f64(in, K, g, H, rot);
            quantize_row_i8(rot, K, xq + m * K, x_scale + m);
        }
        free(in); free(rot);
    }
    free(H);
    return ORACLE_OK;
}

/* ----------------------------------------------------------------- GEMM */

/* acc[m,n] = sum_k xq[m,k] * wq[n,k] ([P1] intro: the matmuls run in int8,
 * weights and activations).  Naive triple loop; the sum is kept in int64 and
 * must fit int32. */
int oracle_gemm_i8(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc) {
    if (!xq || !wq || !acc || M < 0 || N < 0 || K <= 0) return ORACLE_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)xq[m * K + k] * (int64_t)wq[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return bad ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* y[m,n] = bf16_rne(((float)acc * x_scale[m]) * w_scale[n]); output dtype is
 * the original bf16 ([P4] "Quantization metadata": orig_dtype bfloat16). */
int oracle_epilogue(const int32_t *acc, const float *x_scale, const float *w_scale,
                    int64_t M, int64_t N, uint16_t *y) {
    if (!acc || !x_scale || !w_scale || !y || M < 0 || N < 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float a = (float)acc[m * N + n];
            float t = a * x_scale[m];
            float r = t * w_scale[n];
            y[m * N + n] = float_to_bf16_rne(r);
        }
    }
    return ORACLE_OK;
}

/* The whole W8A8 linear: rotate + quantize x, int8 GEMM, rescale to bf16. */
int oracle_w8a8_linear(const uint16_t *x, int64_t M, int64_t K, const int8_t *wq, const float *w_scale,
                       int64_t N, int g, uint16_t *y) {
    if (!x || !wq || !w_scale || !y || M < 0 || N < 0 || K <= 0) return ORACLE_ERR_ARG;
    if (M == 0 || N == 0) return ORACLE_OK;
    int8_t *xq = (int8_t *)malloc((size_t)(M * K));
    float *xs = (float *)malloc(sizeof(float) * (size_t)M);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * N));
    int rc = (xq && xs && acc) ? ORACLE_OK : ORACLE_ERR_ARG;
    if (rc == ORACLE_OK) rc = oracle_rotate_quant(x, M, K, g, xq, xs);
    if (rc == ORACLE_OK) rc = oracle_gemm_i8(xq, wq, M, N, K, acc);
    if (rc == ORACLE_OK) rc = oracle_epilogue(acc, xs, w_scale, M, N, y);
    free(xq); free(xs); free(acc);
    return rc;
}

/* ------------------------------------------------------------------ int4 */

/* Scale for clip candidate i (c = (100 - i) / 100, i = 0..50):
 * s = c * absmax / 7, evaluated as absmax * (100 - i) / 700 in fp64 and
 * rounded to fp32 ([P5] "Format": one F32 scale per row chosen by a clip
 * search per row). */
static float int4_candidate_scale(double amax, int i) {
    return (float)(amax * (double)(100 - i) / 700.0);
}

/* Codes of a row for a given scale: round_half_away(v / s) on the fp64
 * quotient, clamped to [-7, 7] (signed 4-bit codes, [P5] "Format"). */
static void int4_codes(const double *v, int64_t K, float s, int8_t *q) {
    for (int64_t k = 0; k < K; ++k) {
        if (s == 0.0f) { q[k] = 0; continue; }
        double r = round_half_away(v[k] / (double)s);
        if (r > 7.0) r = 7.0;
        if (r < -7.0) r = -7.0;
        q[k] = (int8_t)r;
    }
}

/* Sum of squared reconstruction error of a row, in fp64. */
static double int4_row_error(const double *v, int64_t K, float s, const int8_t *q) {
    double e = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double d = (double)q[k] * (double)s - v[k];
        e += d * d;
    }
    return e;
}

/* Weight preparation, int4: W fp32 [N,K] -> wq4 uint8 [N,K/2] (two signed
 * nibbles per byte, low nibble = even column), scale fp32 [N].
 *   clip_index (may be NULL) receives the winning candidate i (c = 1 - i/100);
 *   errors (may be NULL, [N, 51]) receives every candidate's error;
 *   force_index (may be NULL, [N]) skips the choice: row n takes candidate
 *   force_index[n] (in 0..50) instead of the argmin.  The tests use the last
 *   two to judge a kernel whose choice differs on a near tie. */
int oracle_quantize_weight_i4_ex(const float *w, int64_t N, int64_t K, int g, const int32_t *force_index,
                                 uint8_t *wq4, float *scale, int32_t *clip_index, double *errors) {
    if (!w || !wq4 || !scale || N < 0 || K <= 0 || (K & 1) || !is_pow2(g) || K % g) return ORACLE_ERR_ARG;
    if (force_index)
        for (int64_t n = 0; n < N; ++n)
            if (force_index[n] < 0 || force_index[n] > 50) return ORACLE_ERR_ARG;
    double *H = (double *)malloc(sizeof(double) * (size_t)g * (size_t)g);
    if (!H) return ORACLE_ERR_ARG;
    oracle_hadamard(g, H);
#pragma omp parallel
    {
        double *in = (double *)malloc(sizeof(double) * (size_t)K);
        double *rot = (double *)malloc(sizeof(double) * (size_t)K);
        int8_t *q = (int8_t *)malloc((size_t)K);
        int8_t *best_q = (int8_t *)malloc((size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) in[k] = (double)w[n * K + k];
            rotate_row_f64(in, K, g, H, rot);
            double amax = 0.0;
            for (int64_t k = 0; k < K; ++k)
                if (fabs(rot[k]) > amax) amax = fabs(rot[k]);
            int best_i = 0;
            double best_err = 0.0;
            float best_s = 0.0f;
            for (int i = 0; i <= 50; ++i) {
                float s = int4_candidate_scale(amax, i);
                int4_codes(rot, K, s, q);
                double e = int4_row_error(rot, K, s, q);
                if (errors) errors[n * 51 + i] = e;
                const int take = force_index ? (i == force_index[n]) : (i == 0 || e < best_err);
                if (take) {
                    best_err = e; best_i = i; best_s = s;
                    memcpy(best_q, q, (size_t)K);
                }
            }
            scale[n] = best_s;
            if (clip_index) clip_index[n] = best_i;
            for (int64_t j = 0; j < K / 2; ++j) {
                uint8_t lo = (uint8_t)best_q[2 * j] & 0x0fu;
                uint8_t hi = (uint8_t)best_q[2 * j + 1] & 0x0fu;
                wq4[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
            }
        }
        free(in); free(rot); free(q); free(best_q);
    }
    free(H);
    return ORACLE_OK;
}

/* The clip search as defined: every row takes its argmin candidate. */
int oracle_quantize_weight_i4(const float *w, int64_t N, int64_t K, int g, uint8_t *wq4, float *scale,
                              int32_t *clip_index) {
    return oracle_quantize_weight_i4_ex(w, N, K, g, NULL, wq4, scale, clip_index, NULL);
}

/* Packed int4 [N,K/2] -> int8 codes [N,K]: each nibble read as a signed
 * 4-bit two's-complement number (-8..7). */
int oracle_unpack_i4(const uint8_t *wq4, int64_t N, int64_t K, int8_t *wq) {
    if (!wq4 || !wq || N < 0 || K <= 0 || (K & 1)) return ORACLE_ERR_ARG;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = wq4[n * (K / 2) + j];
            int lo = b & 0x0f, hi = b >> 4;
            wq[n * K + 2 * j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            wq[n * K + 2 * j + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
    }
    return ORACLE_OK;
}

/* The W4A8 linear: int4 weights unpacked, then exactly the W8A8 path
 * ([P5] "Format": computation runs with 8-bit activations). */
int oracle_w4a8_linear(const uint16_t *x, int64_t M, int64_t K, const uint8_t *wq4, const float *w_scale,
                       int64_t N, int g, uint16_t *y) {
    if (!x || !wq4 || !w_scale || !y || M < 0 || N < 0 || K <= 0 || (K & 1)) return ORACLE_ERR_ARG;
    if (M == 0 || N == 0) return ORACLE_OK;
    int8_t *wq = (int8_t *)malloc((size_t)(N * K));
    int rc = wq ? oracle_unpack_i4(wq4, N, K, wq) : ORACLE_ERR_ARG;
    if (rc == ORACLE_OK) rc = oracle_w8a8_linear(x, M, K, wq, w_scale, N, g, y);
    free(wq);
    return rc;
}

/* ------------------------------------------------------------- RMSNorm */

/* The decoder-layer RMSNorm that precedes the quantized linears ([P1] table
 * row "Changed": its weights carry the SmoothQuant scales; "How it was made":
 * the scales are folded into the norm as (1 + w) / s - 1, i.e. the norm
 * multiplies by (1 + w)).  Per row of x bf16 [M,K]:
 *   ms = (float)(sum_k x_k^2 / K)   (the sum in fp64: every x_k^2 of a bf16
 *                                    value is exact there)
 *   r  = 1 / sqrt(ms + eps)         (fp32, each operation rounded)
 *   y_k = bf16_rne((x_k * r) * (1 + w_k))  (fp32, in this order)
 * The output is bf16, the activation dtype the linear's input has.  Every
 * step is fp32 except the sum, so a GPU that accumulates in fp64 as well
 * reaches the same bf16 values. */
int oracle_rmsnorm_bf16(const uint16_t *x, const float *w, float eps, int64_t M, int64_t K, uint16_t *y) {
    if (!x || !w || !y || M < 0 || K <= 0 || !(eps >= 0.0f)) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double v = bf16_bits_to_double(xr[k]);
            ss += v * v;
        }
        const float ms = (float)(ss / (double)K);
        const float r = 1.0f / sqrtf(ms + eps);
        for (int64_t k = 0; k < K; ++k) {
            const float t = (float)bf16_bits_to_double(xr[k]) * r;
            const float u = t * (1.0f + w[k]);
            y[m * K + k] = float_to_bf16_rne(u);
        }
    }
    return ORACLE_OK;
}

/* RMSNorm followed by the activation rotate + quantization of its bf16
 * output: what the linear after a norm sees. */
int oracle_rmsnorm_rotate_quant(const uint16_t *x, const float *w, float eps, int64_t M, int64_t K, int g,
                                int8_t *xq, float *x_scale, uint16_t *y) {
    int rc = oracle_rmsnorm_bf16(x, w, eps, M, K, y);
    if (rc == ORACLE_OK) rc = oracle_rotate_quant(y, M, K, g, xq, x_scale);
    return rc;
}

/* ------------------------------------------------ weight-only dequant path */

/* The weight-only runtime mode ([P1] file table, row "Matmul": a mode that
 * expands the codes back into a bf16 weight and multiplies in bf16; [P2]
 * loads the checkpoints through that dequant path).  A stored row holds the
 * codes of the ROTATED weight row, so the weight is recovered by undoing the
 * rotation: W^ = (wq * s_w) * H^-1, and H^-1 = H (the normalised Sylvester
 * matrix is symmetric and orthogonal).  H is the +-1 Sylvester pattern times
 * 1/sqrt(g), so per group of g columns the product is evaluated as
 *   t_k      = sum_j code_j * sign(H[j][k])   (an integer, |t| <= 256 * 128:
 *                                              exact in fp64, in any order)
 *   u_k      = (t_k * s_w[n]) * H[0][0] + 0   (t * s_w exact in fp64; one
 *                                              rounding by 1/sqrt(g), none for
 *                                              even log2(g); + 0 makes a zero
 *                                              result +0, as the sum of the
 *                                              dense product's terms is)
 *   W^[n][k] = bf16_rne((float)u_k)           (rounded to fp32, the scale's
 *                                              precision, then to bf16)
 * This is the product itself, exact but for the one irrational constant: an
 * fp64 dense product would round every term by 1/sqrt(g) for odd log2(g) and
 * leave a residue of order 1e-19 where the exact value is 0.
 * int4 rows are unpacked to their codes first (oracle_unpack_i4). */
int oracle_dequantize_weight(const int8_t *wq, const float *w_scale, int64_t N, int64_t K, int g, uint16_t *w_out) {
    if (!wq || !w_scale || !w_out || N < 0 || K <= 0 || !is_pow2(g) || K % g) return ORACLE_ERR_ARG;
    double *H = (double *)malloc(sizeof(double) * (size_t)g * (size_t)g);
    if (!H) return ORACLE_ERR_ARG;
    oracle_hadamard(g, H);
    const double norm = H[0];
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const int8_t *q = wq + n * K;
        const double s = (double)w_scale[n];
        for (int64_t base = 0; base < K; base += g) {
            for (int k = 0; k < g; ++k) {
                double t = 0.0;
                for (int j = 0; j < g; ++j)
                    t += (H[(int64_t)j * g + k] > 0.0 ? 1.0 : -1.0) * (double)q[base + j];
                const double u = (t * s) * norm + 0.0;
                w_out[n * K + base + k] = float_to_bf16_rne((float)u);
            }
        }
    }
    free(H);
    return ORACLE_OK;
}

/* The bf16 matmul of the dequant path: y[m][n] = bf16_rne((float)s) with
 * s = sum_k x[m][k] * w[n][k] accumulated in fp64 in k order (each product
 * of two bf16 values is exact in fp64), rounded to fp32 and then to bf16. */
int oracle_gemm_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K, uint16_t *y) {
    if (!x || !w || !y || M < 0 || N < 0 || K <= 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += bf16_bits_to_double(x[m * K + k]) * bf16_bits_to_double(w[n * K + k]);
            y[m * N + n] = float_to_bf16_rne((float)acc);
        }
    }
    return ORACLE_OK;
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel regions that follow (n >= 1); the CPU baseline
 * times the oracle on all cores and on one. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
