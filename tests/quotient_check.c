/*
 * Host check of the GPU kernels' per-element quotient (test code only).
 *
 * The quantizers need v = RN32(x / s) exactly (the code of x is E4M3(v), or RNE(v) for the
 * INT8 variant).  On the GPU each group computes s = RN32(amax / D), D = 448 for FP8 (the
 * default) or 127 for INT8 (first argument), and r = RN32(1 / s) once, and each element
 * then takes three operations (P. Markstein, IBM J. Res. Dev. 34(1), 1990):
 *     q = RN(x * r);  e = RN(q * s - x) [one FMA];  v = RN(-e * r + q) [one FMA]
 * Groups with 0 < s < 2^-100 first scale both x and s by m = 2^64 (exact: a power of two
 * applied to a bf16 x and to s, nothing overflows), i.e. they run the same three operations
 * on x*m with sq = s*m and r = RN32(1 / sq).  A group with s == 0 (amax == 0, every x is +-0)
 * uses r = 0, which yields the signed zero of x.  This program
 * replays exactly those binary32 operations for EVERY pair (amax, x) of finite bf16 values
 * with |x| <= amax and compares v with the IEEE binary32 division x / s:
 *   - where |x / s| > 2^-10 (the code is not +-0), v must equal x / s bit for bit;
 *   - where |x / s| <= 2^-10 (the code is +-0: 2^-10 is the tie between 0 and 2^-9 and goes
 *     to the even code 0), v must also be <= 2^-10 in magnitude and carry the same sign.
 * The second case is needed only where the residual q*s - x falls below the binary32
 * subnormal range (x itself tiny), which leaves v off by an ulp far below 2^-10.
 * It prints the pair count, the code-level mismatches (0 expected) and, for information, the
 * pairs where v is not bit-identical to x / s.
 *
 * Build at -O0: gcc -O2 folds the negations across the two FMAs, which is not sign-of-zero
 * safe (x = -0 then yields +0); the GPU compiler keeps the operations as written.
 * gcc -O0 -ffp-contract=off -fopenmp [-mfma] quotient_check.c -lm;  ./a.out [D]
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t b)
{
    uint32_t u = b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

int main(int argc, char **argv)
{
    const float div = argc > 1 ? (float)atof(argv[1]) : 448.0f;
    long long mismatches = 0, pairs = 0, inexact = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : mismatches, pairs, inexact)
    for (uint32_t ab = 0; ab < 0x7F80u; ++ab) {          /* every finite amax >= 0 */
        const float amax = bf16(ab);
        const float s = amax / div;
        const float m = (s > 0.0f && s < 0x1p-100f) ? 0x1p64f : 1.0f;
        const float sq = s * m;
        const float r = sq == 0.0f ? 0.0f : 1.0f / sq;
        for (uint32_t xb = 0; xb < 0x10000u; ++xb) {
            if ((xb & 0x7F80u) == 0x7F80u)
                continue;                                 /* Inf / NaN */
            if ((xb & 0x7FFFu) > ab)
                continue;                                 /* |x| > amax: not in this group */
            const float x = bf16(xb);
            const float xm = x * m;
            const float q = xm * r;
            const float e = fmaf(q, sq, -xm);
            const float v = fmaf(-e, r, q);
            const float ref = s == 0.0f ? x : x / s;
            ++pairs;
            int ok;
            if (fabsf(ref) > 0x1p-10f)
                ok = bits(v) == bits(ref);
            else
                ok = fabsf(v) <= 0x1p-10f && (bits(v) >> 31) == (bits(ref) >> 31);
            mismatches += !ok;
            inexact += bits(v) != bits(ref);
        }
    }
    printf("divisor %g pairs %lld mismatches %lld not_bit_identical %lld\n", (double)div, pairs,
           mismatches, inexact);
    return mismatches != 0;
}
