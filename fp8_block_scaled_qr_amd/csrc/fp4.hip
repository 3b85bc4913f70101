// 4-bit weights for gfx950: quantization to E2M1 elements with an E4M3 scale per 16 elements
// and an fp32 tensor scale, and the GEMM of bf16 activations with those weights.
//
// The format follows the QeRL notes (4-bit floats with two-level scaling: FP8 E4M3 block
// scales and an FP32 tensor scale, used for the rollout's weights):
//   t = RN32(amax / 2688)                (2688 = 448 * 6: block scales then fit E4M3)
//   block scale code = E4M3(RN32(amax_b / RN32(6 t)))        (blocks of 16 along a row)
//   element code = E2M1(RN32(x / RN32(dq(block scale) * t)))  (nearest, ties to even, <= 6)
// Element 2j of a row sits in the low nibble of byte j.
//
// gfx950's FP4 MFMA takes power-of-two block scales, which these E4M3 scales are not, so the
// GEMM dequantizes in registers instead: v_cvt_scalef32_pk_f32_fp4 with scale 1 gives the
// E2M1 values exactly, times the block scale is exact in binary32 (at most 6 significant
// bits), and truncating that to bf16 is exact too; bf16 MFMAs then accumulate in fp32 and the
// tensor scale is applied once, in the epilogue.
#include "qr_device.h"
#include "qr_internal.h"

namespace qr {

namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kAmaxGrid = kNvfp4Partials;   // partial maxima (one per workgroup of the first pass)

__device__ __forceinline__ uint32_t absmax8_16(const uint4 &v)
{
    return umax(umax(absmax2(v.x), absmax2(v.y)), umax(absmax2(v.z), absmax2(v.w)));
}

// Pass 1: each workgroup's maximum |w| (as a 15-bit bf16 magnitude pattern) over a grid-stride
// share of the 16-byte chunks.
__global__ __launch_bounds__(256) void k_nvfp4_amax(const uint16_t *__restrict__ w, int64_t n,
                                                    int64_t k, int64_t ld,
                                                    uint32_t *__restrict__ partial)
{
    __shared__ uint32_t red[4];
    const int64_t cpr = k / 8, total = n * cpr;
    uint32_t m = 0;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * 256) {
        const int64_t r = c / cpr, col = (c - r * cpr) * 8;
        m = umax(m, absmax8_16(*reinterpret_cast<const uint4 *>(w + r * ld + col)));
    }
    for (int o = 32; o >= 1; o >>= 1)
        m = umax(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        partial[blockIdx.x] = umax(umax(red[0], red[1]), umax(red[2], red[3]));
}

// E2M1 code of a binary32 quotient: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even
// code (the midpoints 0.25, 1.25, 2.5, 5 go down, 0.75, 1.75, 3.5 up), saturating at 6; the
// sign of v is kept.
__device__ __forceinline__ uint32_t e2m1_code(float v)
{
    const float a = fabsf(v);
    const uint32_t idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                         (a >= 3.5f) + (a > 5.0f);
    return idx | ((__float_as_uint(v) >> 28) & 8u);
}

// Pass 2: every workgroup reduces the partial maxima to t, then a thread encodes one block of
// 16 elements at a time (two 16-byte loads, one 8-byte code store, one scale byte).
__global__ __launch_bounds__(256) void k_nvfp4_quant(const uint16_t *__restrict__ w, int64_t n,
                                                     int64_t k, int64_t ld,
                                                     const uint32_t *__restrict__ partial,
                                                     int npartial, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ bscale,
                                                     float *__restrict__ tscale)
{
    __shared__ uint32_t red[4];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += 256)
        m = umax(m, partial[i]);
    for (int o = 32; o >= 1; o >>= 1)
        m = umax(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    const float t = __fdiv_rn(__uint_as_float(m << 16), 2688.0f);
    const float u = __fmul_rn(6.0f, t);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *tscale = t;

    const int64_t bpr = k / 16, total = n * bpr;
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < total;
         b += (int64_t)gridDim.x * 256) {
        const int64_t r = b / bpr, bc = b - r * bpr;
        const uint16_t *src = w + r * ld + 16 * bc;
        const uint4 v0 = *reinterpret_cast<const uint4 *>(src);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(src + 8);
        const uint32_t ab = umax(absmax8_16(v0), absmax8_16(v1));
        uint32_t sb = 0;
        float e = 0.0f;
        if (t > 0.0f) {
            // below 464, so the conversion's saturation of [448, 464) to 448 is all we need
            sb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                     __fdiv_rn(__uint_as_float(ab << 16), u), 0.0f, 0, false) & 0xFFu;
            e = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)sb, 0), t);
        }
        uint32_t out[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float x = bf16_elem(i < 8 ? v0 : v1, i & 7);
            const uint32_t c = e != 0.0f ? e2m1_code(__fdiv_rn(x, e))
                                         : ((__float_as_uint(x) >> 28) & 8u);
            out[i >> 3] |= c << (4 * (i & 7));
        }
        *reinterpret_cast<uint2 *>(codes + r * (k / 2) + 8 * bc) = make_uint2(out[0], out[1]);
        bscale[r * bpr + bc] = (uint8_t)sb;
    }
}

// 8 bf16 weights (one dword of codes, elements 0..7) scaled by a block scale: the FP4
// conversion with scale 1 is exact, the product with the E4M3 scale is exact in binary32,
// and the bf16 is its upper half (exact).
template <int J>
__device__ __forceinline__ uint32_t dequant2(uint32_t codes8, float sc)
{
    const v2f f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes8, 1.0f, J);   // byte J
    return (__float_as_uint(f[0] * sc) >> 16) | (__float_as_uint(f[1] * sc) & 0xFFFF0000u);
}

__device__ __forceinline__ v8bf dequant8(uint32_t codes8, float sc)
{
    return __builtin_bit_cast(v8bf, make_uint4(dequant2<0>(codes8, sc), dequant2<1>(codes8, sc),
                                               dequant2<2>(codes8, sc), dequant2<3>(codes8, sc)));
}

// Y[m, n] = t * sum_k X[m, k] * W[n, k], X bf16 [M, K], W in 4-bit codes.  A workgroup owns 64
// rows of W (4 waves x 16) and 64 rows of X (grid y); a K step is 128.
//   X: the step's 64 x 128 tile (16 KB) is staged in LDS (two buffers, register staging); row
//      r's 16-byte chunk c sits in slot c ^ (r % 16).
//   W: lane (n = l % 16, q = l / 16) loads the 32 codes of K range [32 q, 32 q + 32) of its row
//      (16 bytes) and their 2 block scales, one step ahead.
// MFMA s (0..3) of a step covers K offsets 32 q + 8 s .. + 7 in lane group q, for both
// operands; four 16x16x32 bf16 MFMAs per 16-row block of X.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_gemm_w4a16(const uint16_t *__restrict__ X,
                                                    const uint8_t *__restrict__ codes,
                                                    const uint8_t *__restrict__ bscale,
                                                    const float *__restrict__ tscale, int64_t M,
                                                    int64_t N, int64_t K, void *__restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][64 * 256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lq = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 64, m0 = (int64_t)blockIdx.y * 64;
    const int64_t nrow = n0 + 16 * wave + ln;
    const bool nok = nrow < N;
    const int64_t steps = K / 128;

    // X staging: thread tid takes row tid / 4, chunks 4 (tid % 4) .. + 3 of the 16 in a row
    const int xr = tid >> 2, xc0 = 4 * (tid & 3);
    const bool xok = m0 + xr < M;
    const uint16_t *xsrc = X + (m0 + xr) * K + 8 * xc0;
    auto xload = [&](int64_t s, uint4 (&v)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = xok ? *reinterpret_cast<const uint4 *>(xsrc + 128 * s + 8 * j)
                       : make_uint4(0, 0, 0, 0);
    };
    auto xstore = [&](int buf, const uint4 (&v)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint4 *>(&xs[buf][xr * 256 + (((xc0 + j) ^ (xr & 15)) << 4)]) = v[j];
    };
    const uint8_t *wsrc = codes + nrow * (K / 2) + 16 * lq;
    const uint8_t *ssrc = bscale + nrow * (K / 16) + 2 * lq;
    auto wload = [&](int64_t s, uint4 &c, uint32_t &sc2) {
        if (nok) {
            c = *reinterpret_cast<const uint4 *>(wsrc + 64 * s);
            sc2 = *reinterpret_cast<const uint16_t *>(ssrc + 8 * s);
        } else {
            c = make_uint4(0, 0, 0, 0);
            sc2 = 0;
        }
    };

    v4f acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 xv[4], wc, wcn;
    uint32_t ws2 = 0, wsn = 0;
    if (steps > 0) {
        xload(0, xv);
        xstore(0, xv);
        wload(0, wc, ws2);
    }
    __syncthreads();
    for (int64_t s = 0; s < steps; ++s) {
        const int buf = (int)(s & 1);
        const bool more = s + 1 < steps;
        if (more) {
            xload(s + 1, xv);
            wload(s + 1, wcn, wsn);
        }
        const float sc0 = __builtin_amdgcn_cvt_f32_fp8((int)(ws2 & 0xFFu), 0);
        const float sc1 = __builtin_amdgcn_cvt_f32_fp8((int)(ws2 >> 8), 0);
        const v8bf wf[4] = {dequant8(wc.x, sc0), dequant8(wc.y, sc0), dequant8(wc.z, sc1),
                            dequant8(wc.w, sc1)};
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int row = 16 * mb + ln;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const v8bf xf = *reinterpret_cast<const v8bf *>(
                    &xs[buf][row * 256 + (((4 * lq + t) ^ (row & 15)) << 4)]);
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[t], xf, acc[mb], 0, 0, 0);
            }
        }
        if (more) {
            xstore(buf ^ 1, xv);   // read last in step s - 1, before the barrier that ended it
            wc = wcn;
            ws2 = wsn;
        }
        __syncthreads();
    }

    // epilogue: lane holds Y[m = row l % 16 of block mb][n .. n + 3]
    const float t = *tscale;
    const int64_t n = n0 + 16 * wave + 4 * lq;
    const bool vec_ok = (N & 3) == 0 && n + 3 < N;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int64_t m = m0 + 16 * mb + ln;
        if (m >= M)
            continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = acc[mb][r] * t;
        if (!OUT_BF16) {
            float *c = reinterpret_cast<float *>(Y) + m * N + n;
            if (vec_ok) {
                *reinterpret_cast<float4 *>(c) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        c[r] = v[r];
            }
        } else {
            uint16_t *c = reinterpret_cast<uint16_t *>(Y) + m * N + n;
            if (vec_ok) {
                *reinterpret_cast<uint2 *>(c) =
                    make_uint2(f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16),
                               f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        c[r] = (uint16_t)f32_to_bf16(v[r]);
            }
        }
    }
}

}  // namespace

hipError_t launch_quant_nvfp4(const uint16_t *w, int64_t n, int64_t k, int64_t ld, uint8_t *codes,
                              uint8_t *bscale, float *tscale, uint32_t *partial,
                              hipStream_t stream)
{
    const int64_t chunks = n * (k / 8);
    int64_t g = (chunks + 255) / 256;
    if (g > kAmaxGrid)
        g = kAmaxGrid;
    if (g < 1)
        g = 1;
    k_nvfp4_amax<<<(unsigned)g, 256, 0, stream>>>(w, n, k, ld, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    int64_t g2 = (n * (k / 16) + 255) / 256;
    if (g2 > 4096)
        g2 = 4096;
    if (g2 < 1)
        g2 = 1;
    k_nvfp4_quant<<<(unsigned)g2, 256, 0, stream>>>(w, n, k, ld, partial, (int)g, codes, bscale,
                                                     tscale);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a16(bool out_bf16, const uint16_t *X, const uint8_t *codes,
                             const uint8_t *bscale, const float *tscale, int64_t M, int64_t N,
                             int64_t K, void *Y, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    if (out_bf16)
        k_gemm_w4a16<true><<<grid, 256, 0, stream>>>(X, codes, bscale, tscale, M, N, K, Y);
    else
        k_gemm_w4a16<false><<<grid, 256, 0, stream>>>(X, codes, bscale, tscale, M, N, K, Y);
    return hipGetLastError();
}

}  // namespace qr
