/*
 * Host check of the GPU UAQ fold's per-element rounding (test code only).
 *
 * The fold writes RN_bf16(w / s) for a bf16 weight w and a binary32 scale s > 0: the exact
 * quotient rounded once to bf16, nearest, ties to even.  The GPU takes one of two routes per
 * element:
 *   fast:  r = RN32(1 / s) once per column; q = RN32(|w| * r); where w, q and s lie in safe
 *          exponent ranges, |w| / s rounds to lo = q truncated to bf16 or to lo + 1 bf16 ulp
 *          (q is within ~2 binary32 ulps of |w| / s), and the sign of the FMA residual
 *          |w| - m * s against their midpoint m picks one;
 *   slow:  the binary64 quotient rounded to 8 significant bits.
 * This program replays both routes in binary32/binary64 exactly as the kernel writes them and
 * compares each result with an exact integer evaluation of RN_bf16(w / s) (long division of
 * the significands, remainder as sticky bit), for every finite bf16 w against
 *   - 4096 scales s ~ U(1.5, 4) (the UAQ range),
 *   - 4096 scales with uniformly random positive finite bit patterns (all exponents,
 *     subnormals included: the slow route and the overflow / underflow ends),
 *   - 48 scales per w that put |w| / s within a few binary32 ulps of a bf16 midpoint
 *     (s = RN32(|w| / m) and its neighbours), where the fast route's decision is closest.
 * It prints the pair count, the mismatches (0 expected), how many pairs took each route and
 * how many fast decisions were close (|residual| < 2^-20 |w|).
 *
 * gcc -O1 -ffp-contract=off -fno-fast-math -fopenmp [-mfma] fold_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f32(uint32_t u)
{
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

/* Exact RN_bf16(w / s), w a finite bf16 (bit pattern), s a positive finite binary32. */
static uint16_t exact_fold(uint32_t wb, float s)
{
    const uint16_t sign = wb & 0x8000u;
    const uint32_t ew = (wb >> 7) & 0xFFu, mw = wb & 0x7Fu;
    if (ew == 0 && mw == 0)
        return sign;
    const uint64_t Mw = ew ? (mw | 0x80u) : mw;            /* w = Mw 2^Xw */
    const int Xw = (ew ? (int)ew : 1) - 127 - 7;
    const uint32_t sb = bits(s), es = sb >> 23, ms = sb & 0x7FFFFFu;
    const uint64_t Ms = es ? (ms | 0x800000u) : ms;         /* s = Ms 2^Xs */
    const int Xs = (es ? (int)es : 1) - 127 - 23;
    const uint64_t N = Mw << 40, Q = N / Ms, R = N % Ms;    /* w/s = (Q + R/Ms) 2^X */
    const int X = Xw - Xs - 40;
    const int L = 64 - __builtin_clzll(Q);                  /* Q >= 2^16: Mw >= 1, Ms < 2^24 */
    int e = L - 1 + X;                                      /* w/s in [2^e, 2^(e+1)) */
    if (e < -126)
        e = -126;                                           /* bf16 subnormal step 2^-133 */
    const int sh = e - 7 - X;                               /* bits of Q below 2^(e-7) */
    uint64_t kept;
    if (sh >= 64) {
        kept = 0;                                           /* w/s < 2^(e-7-16): rounds to 0 */
    } else {
        kept = Q >> sh;
        const uint64_t rest = Q & ((1ull << sh) - 1), half = 1ull << (sh - 1);
        if (rest > half || (rest == half && (R != 0 || (kept & 1))))
            ++kept;
    }
    if (kept == 256) {
        kept = 128;
        ++e;
    }
    if (kept < 128)
        return sign | (uint16_t)kept;                       /* subnormal or zero */
    if (e + 127 >= 255)
        return sign | 0x7F80u;                              /* overflow to infinity */
    return sign | (uint16_t)(((uint32_t)(e + 127) << 7) | (kept & 0x7Fu));
}

/* The kernel's slow route. */
static uint16_t slow_fold(uint32_t wb, float s)
{
    const float wv = f32(wb << 16);
    const double d = (double)wv / (double)s;
    const double a = fabs(d);
    double rv = 0.0;
    if (a != 0.0) {
        int e = ilogb(a);
        if (e < -126)
            e = -126;
        rv = ldexp(rint(ldexp(a, 7 - e)), e - 7);
    }
    return (uint16_t)((bits((float)rv) >> 16) | (wb & 0x8000u));
}

/* The kernel's fast route; *slow is set where the kernel falls back to the slow route. */
static uint32_t fast_fold(uint32_t wb, float s, float r, int col_ok, int *slow, float *resid)
{
    const float a = f32((wb & 0x7FFFu) << 16);
    const uint32_t qb = bits(a * r);
    const uint32_t ew = (wb >> 7) & 0xFFu, eq = qb >> 23;
    const uint32_t lo = qb & 0xFFFF0000u;
    const float d = fmaf(-f32(lo | 0x8000u), s, a);
    const uint32_t up = d > 0.0f ? 1u : (d == 0.0f ? (lo >> 16) & 1u : 0u);
    const int zero = (wb & 0x7FFFu) == 0;
    const int ok = col_ok && ew >= 37u && eq - 27u <= 220u;
    *slow = !(ok || zero);
    *resid = zero ? 1.0f : fabsf(d) / a;
    return zero ? wb : (((lo >> 16) + up) | (wb & 0x8000u));
}

static uint64_t rng_state;

static uint32_t rnd(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng_state >> 32);
}

#define NS_FIXED 8192
#define NS_ADV 48

int main(void)
{
    static float fixed[NS_FIXED];
    rng_state = 12345;
    for (int i = 0; i < NS_FIXED / 2; ++i)
        fixed[i] = 1.5f + 2.5f * (float)((rnd() >> 8) * 0x1p-24);
    for (int i = NS_FIXED / 2; i < NS_FIXED; ++i) {
        uint32_t b;
        do
            b = rnd() & 0x7FFFFFFFu;
        while (b == 0 || (b >> 23) == 0xFF);
        fixed[i] = f32(b);
    }
    long long pairs = 0, mismatches = 0, slow_n = 0, fast_n = 0, close_n = 0;
#pragma omp parallel for schedule(dynamic, 256) \
    reduction(+ : pairs, mismatches, slow_n, fast_n, close_n)
    for (uint32_t wb = 0; wb < 0x10000u; ++wb) {
        if ((wb & 0x7F80u) == 0x7F80u)
            continue;                                       /* Inf / NaN */
        float ss[NS_FIXED + NS_ADV];
        memcpy(ss, fixed, sizeof fixed);
        int ns = NS_FIXED;
        const double aw = fabs((double)f32(wb << 16));
        uint64_t st = 0x9E3779B97F4A7C15ull * (wb + 1);
        for (int j = 0; j < 64 && ns < NS_FIXED + NS_ADV && aw > 0.0; ++j) {
            st = st * 6364136223846793005ull + 1442695040888963407ull;
            const double t = aw / (1.5 + 2.5 * (double)(st >> 11) * 0x1p-53);
            const double ulp = ldexp(1.0, ilogb(t) - 7);
            const double m = (floor(t / ulp) + 0.5) * ulp;  /* the bf16 midpoint below t */
            const float s0 = (float)(aw / m);
            for (int k = -1; k <= 1 && ns < NS_FIXED + NS_ADV; ++k) {
                const float sk = f32(bits(s0) + (uint32_t)k);
                if (sk > 0.0f && isfinite(sk))
                    ss[ns++] = sk;
            }
        }
        for (int i = 0; i < ns; ++i) {
            const float s = ss[i];
            const float r = 1.0f / s;
            const int col_ok = (bits(s) >> 23) - 7u <= 240u;
            int slow;
            float resid;
            uint32_t got = fast_fold(wb, s, r, col_ok, &slow, &resid);
            if (slow) {
                got = slow_fold(wb, s);
                ++slow_n;
            } else {
                ++fast_n;
                close_n += resid < 0x1p-20f;
            }
            ++pairs;
            mismatches += got != exact_fold(wb, s);
        }
    }
    printf("pairs %lld mismatches %lld fast %lld slow %lld close %lld\n", pairs, mismatches,
           fast_n, slow_n, close_n);
    return mismatches != 0;
}
