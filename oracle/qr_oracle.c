/*
 * Reference oracle for the fine-grained FP8 quantize-and-multiply of a linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls this file:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no source, header, table or helper with the HIP library.
 *
 * What it computes, and where the pages define it:
 *   - "Jet-RL: Enabling On-Policy FP8 Reinforcement Learning with Unified Training and
 *     Rollout Precision Flow" (arXiv 2601.14243v1) notes, section "细粒度 GEMM 量化方案"
 *     (fine-grained GEMM quantization scheme, around the paper's Figure 6): weights are
 *     quantized per 128x128 block, activations and gradients per 1x128 group; FProp takes the
 *     activation 1x128 row-major and the weight 128x128 "column-major"; DGrad reuses the
 *     FProp configuration; WGrad takes its first operand 1x128 and its second 128x1.
 *   - "QuRL: Efficient Reinforcement Learning with Quantized Rollout" (ICLR 2026) notes,
 *     section "关键设计 1. 更新感知量化 (UAQ)": the invariance WX = (W/s)(sX), s applied per
 *     column of W and per row of the preceding activation, folded into the norm gain once
 *     before training.
 *
 * Readings where the pages are silent (the pages say only "FP8"):
 *   - FP8 is OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; largest finite 448;
 *     S.1111.111 is NaN; no infinities; subnormals are M * 2^-9.
 *   - A group's scale is s = RN32(amax / 448), one IEEE binary32 division; amax is exact.
 *   - An element's code is E4M3(RN32(x / s)) with round-to-nearest-even and saturation to
 *     +-448.  The sign of zero is kept.  amax == 0 gives s == 0 and every code is the
 *     signed zero of x.
 *   - A trailing partial group takes amax over the elements present.
 *   - Inputs must be finite; a non-finite input makes a quantizer return an error.
 *   - GEMMs are the plain definition: dequantize each operand (code value times its group's
 *     scale) and sum the products in fp64.
 *   - The UAQ fold writes W' = RN_bf16(W / s) (the exact quotient rounded once) and
 *     gain' = RN32(gain * s).
 *   - The norm whose gain carries s (the QuRL notes fold s into it) is the standard RMSNorm,
 *     y = h * gain / sqrt(mean(h^2) + eps), evaluated in binary64 and rounded once to bf16.
 *   - The 4-bit weight path (QeRL notes: NVFP4, 4-bit floats with two-level scaling, FP8 E4M3
 *     block scales and an FP32 tensor scale): E2M1 elements (values 0, 0.5, 1, 1.5, 2, 3, 4, 6,
 *     signed), blocks of 16 consecutive elements along a weight row; t = RN32(amax / (448*6));
 *     block scale code = E4M3(RN32(amax_b / RN32(6 t))); element code = E2M1(RN32(x / e)) with
 *     e = RN32(block scale * t), nearest, ties to the even code, saturating at 6.
 *   - The INT8 variant (QuRL's experiment setup: channel-wise weights, token-wise
 *     activations) is symmetric: one scale per row, s = RN32(amax / 127); the code is the
 *     binary32 quotient RN32(x / s) rounded to the nearest integer (ties to even) and clamped
 *     to [-127, 127]; the GEMM is the exact integer dot product times both row scales.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math; x86-64 SSE
 * arithmetic, so binary32 and binary64 operations are correctly rounded and subnormals kept).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define GROUP 128
#define E4M3_MAX 448.0

/* ---------------------------------------------------------------- scalar helpers */

/* bf16 is the upper half of a binary32; widening is exact. */
float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f32_bits_hi(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* Decode one E4M3 code to its exact value.  Codes 0x7F and 0xFF are NaN. */
double orc_e4m3_decode(uint8_t q)
{
    int sign = q >> 7;
    int e = (q >> 3) & 15;
    int m = q & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);              /* subnormal: m * 2^-9 */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);       /* normal: 2^(e-7) * (1 + m/8) */
    return sign ? -v : v;
}

/* Encode a binary32 value to E4M3: nearest code, ties to the even mantissa, values at or
 * beyond 448 in magnitude saturate to 448, the sign of zero is kept.  NaN input is a caller
 * error (the quantizers reject non-finite input before they get here). */
uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= E4M3_MAX)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range, spacing 2^-9; n == 8 is the smallest normal 2^-6 = code 0x08 */
        double n = rint(ldexp(a, 9));           /* a * 2^9 is exact; rint ties to even */
        return sign | (uint8_t)n;
    }
    int e2;
    frexp(a, &e2);                              /* a = f * 2^e2 with f in [0.5, 1) */
    int e = e2 - 1;                             /* a in [2^e, 2^(e+1)), e in -6..8 */
    double n = rint(ldexp(a, 3 - e));           /* 3 fraction bits: n in [8, 16] */
    if (n == 16.0) {
        n = 8.0;
        e += 1;
    }
    return sign | (uint8_t)(((e + 7) << 3) | ((int)n - 8));
}

/* One group's scale: RN32(amax / 448).  amax is an exact binary32 value. */
float orc_group_scale(float amax)
{
    return amax / 448.0f;
}

/* Code of one element given its group's scale. */
uint8_t orc_quantize_value(float x, float s)
{
    if (s == 0.0f)
        return orc_e4m3_encode(x);              /* amax == 0: x is +-0 */
    float v = x / s;                            /* correctly rounded binary32 quotient */
    return orc_e4m3_encode(v);
}

/* Array forms of the scalar codec, for tests over many values. */
void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(v[i]);
}

void orc_quantize_value_array(const float *x, const float *s, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_quantize_value(x[i], s[i]);
}

/* ---------------------------------------------------------------- quantizers */

static int all_finite_bf16(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            if ((x[r * ld + c] & 0x7F80) == 0x7F80)
                return 0;
    return 1;
}

/* 1x128 groups along each row: q[r, c] (dense, row-major, ld = cols) and
 * s[r, g] with g = c / 128 (dense, ld = ceil(cols/128)).  Returns 0, or -1 on non-finite. */
int orc_quant_rows_1x128(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                         uint8_t *q, float *s)
{
    if (!all_finite_bf16(x, rows, cols, ld))
        return -1;
    int64_t ng = (cols + GROUP - 1) / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * GROUP, c1 = c0 + GROUP < cols ? c0 + GROUP : cols;
            float amax = 0.0f;
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(orc_bf16_to_f32(x[r * ld + c]));
                if (a > amax)
                    amax = a;
            }
            float sc = orc_group_scale(amax);
            s[r * ng + g] = sc;
            for (int64_t c = c0; c < c1; ++c)
                q[r * cols + c] = orc_quantize_value(orc_bf16_to_f32(x[r * ld + c]), sc);
        }
    }
    return 0;
}

/* 128x1 groups down each column (128 consecutive rows of one column), stored transposed:
 * qT[c, r] (dense, ld = rows) and sT[c, g] with g = r / 128 (ld = ceil(rows/128)). */
int orc_quant_cols_128x1_T(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                           uint8_t *qT, float *sT)
{
    if (!all_finite_bf16(x, rows, cols, ld))
        return -1;
    int64_t ng = (rows + GROUP - 1) / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        for (int64_t g = 0; g < ng; ++g) {
            int64_t r0 = g * GROUP, r1 = r0 + GROUP < rows ? r0 + GROUP : rows;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r) {
                float a = fabsf(orc_bf16_to_f32(x[r * ld + c]));
                if (a > amax)
                    amax = a;
            }
            float sc = orc_group_scale(amax);
            sT[c * ng + g] = sc;
            for (int64_t r = r0; r < r1; ++r)
                qT[c * rows + r] = orc_quantize_value(orc_bf16_to_f32(x[r * ld + c]), sc);
        }
    }
    return 0;
}

/* 128x128 blocks: q[n, k] (dense, ld = k) and s[i, j] for block (i, j) = (n/128, k/128)
 * (ld = ceil(k/128)). */
int orc_quant_blocks_128x128(const uint16_t *w, int64_t n, int64_t k, int64_t ld,
                             uint8_t *q, float *s)
{
    if (!all_finite_bf16(w, n, k, ld))
        return -1;
    int64_t nbi = (n + GROUP - 1) / GROUP, nbj = (k + GROUP - 1) / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < nbi; ++bi) {
        for (int64_t bj = 0; bj < nbj; ++bj) {
            int64_t r0 = bi * GROUP, r1 = r0 + GROUP < n ? r0 + GROUP : n;
            int64_t c0 = bj * GROUP, c1 = c0 + GROUP < k ? c0 + GROUP : k;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float a = fabsf(orc_bf16_to_f32(w[r * ld + c]));
                    if (a > amax)
                        amax = a;
                }
            float sc = orc_group_scale(amax);
            s[bi * nbj + bj] = sc;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c)
                    q[r * k + c] = orc_quantize_value(orc_bf16_to_f32(w[r * ld + c]), sc);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- dequantization */

/* Value of a 1x128-row-grouped tensor: out[r, c] = dq(q[r, c]) * s[r, c/128]. */
void orc_dequant_rows(const uint8_t *q, const float *s, int64_t rows, int64_t cols, double *out)
{
    int64_t ng = (cols + GROUP - 1) / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = orc_e4m3_decode(q[r * cols + c]) * (double)s[r * ng + c / GROUP];
}

/* Value of a 128x128-block tensor: out[n, k] = dq(q[n, k]) * s[n/128, k/128]. */
void orc_dequant_blocks(const uint8_t *q, const float *s, int64_t n, int64_t k, double *out)
{
    int64_t nbj = (k + GROUP - 1) / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            out[r * k + c] =
                orc_e4m3_decode(q[r * k + c]) * (double)s[(r / GROUP) * nbj + c / GROUP];
}

/* ---------------------------------------------------------------- products */

/* Y[m, n] = sum_k A[m, k] * B[n, k] and S[m, n] = sum_k |A[m, k] * B[n, k]|, in fp64.
 * Both operands are dense row-major with the contraction index contiguous.  S may be NULL. */
void orc_matmul_nt(const double *A, const double *B, int64_t M, int64_t N, int64_t K,
                   double *Y, double *S)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double y = 0.0, a = 0.0;
            const double *pa = A + m * K, *pb = B + n * K;
            for (int64_t k = 0; k < K; ++k) {
                double p = pa[k] * pb[k];
                y += p;
                a += fabs(p);
            }
            Y[m * N + n] = y;
            if (S)
                S[m * N + n] = a;
        }
}

/* The same sums for a list of (m, n) output positions only. */
void orc_matmul_nt_sampled(const double *A, const double *B, int64_t K, const int64_t *mi,
                           const int64_t *ni, int64_t count, double *Y, double *S)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double y = 0.0, a = 0.0;
        const double *pa = A + mi[i] * K, *pb = B + ni[i] * K;
        for (int64_t k = 0; k < K; ++k) {
            double p = pa[k] * pb[k];
            y += p;
            a += fabs(p);
        }
        Y[i] = y;
        S[i] = a;
    }
}

/* ---------------------------------------------------------------- UAQ fold */

/* Round a binary64 to bf16, nearest, ties to even (bf16 keeps 8 significant bits; its
 * subnormals are multiples of 2^-133).  The argument is the binary64 rounding of w / s with
 * w a bf16 and s a binary32: if that quotient is not itself a bf16 midpoint it lies at
 * least about 2^-33 (relative) away from every midpoint, far more than binary64's 2^-53
 * rounding step, so rounding through binary64 equals rounding the exact quotient once. */
static uint16_t f64_to_bf16_rne(double d)
{
    double a = fabs(d);
    double r = 0.0;
    if (a != 0.0) {
        int e2;
        frexp(a, &e2);                           /* a in [2^(e2-1), 2^e2) */
        int e = e2 - 1;
        if (e < -126)
            e = -126;                            /* bf16 subnormal spacing 2^-133 */
        double ulp = ldexp(1.0, e - 7);
        r = rint(a / ulp) * ulp;                 /* a / ulp is exact; rint ties to even */
    }
    float f = (float)r;                          /* exact: r is a bf16 value (or overflows) */
    uint16_t b = f32_bits_hi(f);
    if (signbit(d))
        b |= 0x8000;
    return b;
}

/* W'[n, k] = RN_bf16(W[n, k] / s[k]); gain[k] = RN32(gain[k] * s[k]) if gain != NULL.
 * s must be finite and positive.  w_out may equal w (in place).  Returns 0, or -1 on a
 * non-finite weight or a non-positive / non-finite s. */
int orc_uaq_fold(const uint16_t *w, int64_t n, int64_t k, int64_t ld, const float *s,
                 uint16_t *w_out, float *gain)
{
    if (!all_finite_bf16(w, n, k, ld))
        return -1;
    for (int64_t c = 0; c < k; ++c)
        if (!(s[c] > 0.0f) || !isfinite(s[c]))
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            double q = (double)orc_bf16_to_f32(w[r * ld + c]) / (double)s[c];
            w_out[r * ld + c] = f64_to_bf16_rne(q);
        }
    if (gain)
        for (int64_t c = 0; c < k; ++c)
            gain[c] = gain[c] * s[c];
    return 0;
}

/* ---------------------------------------------------------------- RMSNorm in front of a linear */

/* y[r, c] = h[r, c] * gain[c] / sqrt(mean_c h[r, c]^2 + eps), per row, in binary64 (relative
 * error below 2^-50); y_exact (may be NULL) receives it and y_bf16 its RN_bf16.  This is the
 * norm whose gain the UAQ fold scales by s; the fused kernel quantizes its bf16 output in
 * 1x128 groups.  Returns 0, or -1 on a non-finite h or gain or a negative / non-finite eps. */
int orc_rmsnorm(const uint16_t *h, int64_t rows, int64_t cols, int64_t ld, const float *gain,
                float eps, double *y_exact, uint16_t *y_bf16)
{
    if (!all_finite_bf16(h, rows, cols, ld) || !(eps >= 0.0f) || !isfinite(eps))
        return -1;
    for (int64_t c = 0; c < cols; ++c)
        if (!isfinite(gain[c]))
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            double x = (double)orc_bf16_to_f32(h[r * ld + c]);
            ss += x * x;
        }
        double inv = 1.0 / sqrt(ss / (double)cols + (double)eps);
        for (int64_t c = 0; c < cols; ++c) {
            double y = (double)orc_bf16_to_f32(h[r * ld + c]) * (double)gain[c] * inv;
            if (y_exact)
                y_exact[r * cols + c] = y;
            y_bf16[r * cols + c] = f64_to_bf16_rne(y);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- INT8 W8A8 variant */

/* One symmetric scale per row (a token of the activation, an output channel of the weight):
 * s[r] = RN32(amax_r / 127), q[r, c] = clamp(RNE(RN32(x[r, c] / s[r])), -127, 127), and 0 for
 * a row with amax == 0.  Returns 0, or -1 on a non-finite input. */
int orc_quant_int8_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int8_t *q,
                        float *s)
{
    if (!all_finite_bf16(x, rows, cols, ld))
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(orc_bf16_to_f32(x[r * ld + c]));
            if (a > amax)
                amax = a;
        }
        float sc = amax / 127.0f;
        s[r] = sc;
        for (int64_t c = 0; c < cols; ++c) {
            int8_t code = 0;
            if (sc != 0.0f) {
                float v = orc_bf16_to_f32(x[r * ld + c]) / sc;
                double n = rint((double)v);            /* nearest integer, ties to even */
                if (n > 127.0)
                    n = 127.0;
                if (n < -127.0)
                    n = -127.0;
                code = (int8_t)n;
            }
            q[r * cols + c] = code;
        }
    }
    return 0;
}

/* Y[m, n] = sa[m] * sb[n] * sum_k A[m, k] * B[n, k]: the integer sum is exact (int64), the
 * scaling in binary64.  Y may be NULL when only the sampled form is used. */
void orc_gemm_int8(const int8_t *A, const float *sa, const int8_t *B, const float *sb, int64_t M,
                   int64_t N, int64_t K, double *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
            Y[m * N + n] = (double)sa[m] * (double)sb[n] * (double)acc;
        }
}

/* The same at sampled positions (mi[t], ni[t]). */
void orc_gemm_int8_sampled(const int8_t *A, const float *sa, const int8_t *B, const float *sb,
                           int64_t K, const int64_t *mi, const int64_t *ni, int64_t count,
                           double *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k)
            acc += (int64_t)A[mi[t] * K + k] * (int64_t)B[ni[t] * K + k];
        Y[t] = (double)sa[mi[t]] * (double)sb[ni[t]] * (double)acc;
    }
}

/* ---------------------------------------------------------------- 4-bit (NVFP4-style) weights */

static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(uint8_t c)
{
    double m = E2M1_MAG[c & 7];
    return (c & 8) ? -m : m;
}

/* Nearest E2M1 magnitude, ties to the code with an even mantissa bit (even code), saturating
 * at 6; the sign of v is kept (a negative v that rounds to 0 gives the code 8, -0). */
uint8_t orc_e2m1_encode(float v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0)
        return sign | 7;                          /* saturate (distances lose meaning far out) */
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        double dc = fabs(a - E2M1_MAG[c]), db = fabs(a - E2M1_MAG[best]);
        if (dc < db || (dc == db && (c & 1) == 0))
            best = c;
    }
    return sign | (uint8_t)best;
}

/* w [n, k] -> codes [n, k/2] (element 2j in the low nibble of byte j), block scales
 * [n, k/16] (E4M3 codes), tensor scale *t.  k % 16 == 0.  Returns 0, or -1 on a non-finite
 * input or a bad k. */
int orc_quant_nvfp4(const uint16_t *w, int64_t n, int64_t k, int64_t ld, uint8_t *codes,
                    uint8_t *bscale, float *t_out)
{
    if (k % 16 != 0 || !all_finite_bf16(w, n, k, ld))
        return -1;
    float amax = 0.0f;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            float a = fabsf(orc_bf16_to_f32(w[r * ld + c]));
            if (a > amax)
                amax = a;
        }
    float t = amax / 2688.0f;
    *t_out = t;
    float u = 6.0f * t;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 16; ++b) {
            float ab = 0.0f;
            for (int64_t c = 16 * b; c < 16 * b + 16; ++c) {
                float a = fabsf(orc_bf16_to_f32(w[r * ld + c]));
                if (a > ab)
                    ab = a;
            }
            uint8_t sb = t > 0.0f ? orc_e4m3_encode(ab / u) : 0;
            bscale[r * (k / 16) + b] = sb;
            float e = (float)orc_e4m3_decode(sb) * t;
            for (int64_t c = 16 * b; c < 16 * b + 16; c += 2) {
                uint8_t c0 = 0, c1 = 0;
                float x0 = orc_bf16_to_f32(w[r * ld + c]), x1 = orc_bf16_to_f32(w[r * ld + c + 1]);
                if (e != 0.0f) {
                    c0 = orc_e2m1_encode(x0 / e);
                    c1 = orc_e2m1_encode(x1 / e);
                } else {
                    c0 = signbit(x0) ? 8 : 0;
                    c1 = signbit(x1) ? 8 : 0;
                }
                codes[r * (k / 2) + c / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    return 0;
}

/* Y[m, n] = t * sum_k X[m, k] * E2M1(code[n, k]) * E4M3(bscale[n, k/16]), in binary64 (X bf16
 * [M, K]).  With mi/ni non-NULL only those count positions (Y[count]); else all of Y [M, N]. */
void orc_gemm_w4a16(const uint16_t *X, const uint8_t *codes, const uint8_t *bscale, float t,
                    int64_t M, int64_t N, int64_t K, const int64_t *mi, const int64_t *ni,
                    int64_t count, double *Y)
{
    int64_t total = mi ? count : M * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = mi ? mi[i] : i / N, n = ni ? ni[i] : i % N;
        double acc = 0.0;
        for (int64_t kk = 0; kk < K; ++kk) {
            uint8_t byte = codes[n * (K / 2) + kk / 2];
            uint8_t c = (kk & 1) ? (byte >> 4) : (byte & 15);
            double w = orc_e2m1_decode(c) * orc_e4m3_decode(bscale[n * (K / 16) + kk / 16]);
            acc += (double)orc_bf16_to_f32(X[m * K + kk]) * w;
        }
        Y[i] = acc * (double)t;
    }
}
