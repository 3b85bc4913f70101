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

#include <type_traits>

namespace qr {

namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kAmaxGrid = kNvfp4Partials;

// load depth of the 4-bit GEMM (steps ahead) for 16, 32 and 64 rows of X per workgroup
#ifndef QR_W4_D1
#define QR_W4_D1 3
#endif
#ifndef QR_W4_D2
#define QR_W4_D2 2
#endif
#ifndef QR_W4_D4
#define QR_W4_D4 2
#endif
#ifndef QR_W4_M2   // largest M run as 32-row tiles; larger M takes 64-row tiles
#define QR_W4_M2 32
#endif   // partial maxima (one per workgroup of the first pass)

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
        // Element codes.  The code of RN32(x / e) depends only on which interval between two
        // consecutive midpoints (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) that quotient lies in.
        // q = RN32(x * RN32(1 / e)) lies within 1.5 ulp of x / e, hence within 2.5 ulp of
        // RN32(x / e).  Every midpoint has a significand of 1, 1.25, 1.5 or 1.75: its 23
        // fraction bits are a multiple of 2^21.  So unless q's fraction bits lie within 4 of
        // such a multiple (or q is not finite), both quotients sit strictly inside the same
        // interval and q gives the code; the rare rest take the division itself.  The hardware
        // conversion with scale 1 rounds to the nearest E2M1 value, ties to the even code,
        // saturating at 6 and keeping the sign of zero (the rule above, checked on the device).
        const float rcp = e != 0.0f ? __fdiv_rn(1.0f, e) : 0.0f;
        const bool rcp_ok = e != 0.0f && __builtin_isfinite(rcp);
        auto near = [](float q) {
            const uint32_t b = __float_as_uint(q);
            return ((b >> 23) & 0xFFu) == 0xFFu || (((b & 0x7FFFFFu) + 4u) & 0x1FFFFFu) <= 8u;
        };
        // elements 2p and 2p + 1 of vv into byte p of old
        auto pair = [&](auto pc, const uint4 &vv, uint32_t old) -> uint32_t {
            constexpr int P = decltype(pc)::value;
            const float xa = bf16_elem(vv, 2 * P), xb = bf16_elem(vv, 2 * P + 1);
            float qa = xa * rcp, qb = xb * rcp;
            if (!rcp_ok || near(qa) || near(qb)) {
                qa = e != 0.0f ? __fdiv_rn(xa, e) : xa * 0.0f;
                qb = e != 0.0f ? __fdiv_rn(xb, e) : xb * 0.0f;
            }
            return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, qa, qb, 1.0f, P);
        };
        uint32_t out[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 &vv = h == 0 ? v0 : v1;
            uint32_t o = 0u;
            o = pair(std::integral_constant<int, 0>{}, vv, o);
            o = pair(std::integral_constant<int, 1>{}, vv, o);
            o = pair(std::integral_constant<int, 2>{}, vv, o);
            o = pair(std::integral_constant<int, 3>{}, vv, o);
            out[h] = o;
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

// Y[m, n] = t * sum_k X[m, k] * W[n, k], X bf16 [M, K], W in 4-bit codes.  Decode-shaped: the
// weight bytes dominate, so the kernel is built to keep many of them in flight.
//   Workgroup: 64 rows of W (4 blocks of 16) x 16 MB rows of X (grid y).  Its 4 waves split K:
//   wave w takes the 128-wide K steps s = w, w + 4, ... (the waves of a workgroup read adjacent
//   code bytes), and each holds partial sums for the whole 64 x 16 MB tile; the partials are
//   summed through LDS once, at the end.
//   W codes: lane (l % 16, q = l / 16) loads, per block of 16 rows, the 32 codes of K range
//   [32 q, 32 q + 32) of its row (16 bytes) into registers.
//   W block scales: the step's 8 scale bytes of each of the 64 rows go to a per-wave LDS ring
//   by two direct-to-LDS dword loads (lane = row); each lane reads back its 2 bytes per block.
//   X: the step's 16 MB rows x 256 bytes go to the same ring by direct-to-LDS loads of whole
//   lines (4 rows x 256 bytes per instruction), row-major with the 16-byte chunk c of row r at
//   slot c ^ (r % 16); each fragment read back (conflict-free) serves the 4 W blocks.
//   All three run D steps ahead, refilled together at the end of each step: loads retire in
//   order, so a stream kept shallower than another would cap the other's depth at its own.
//   The ring's wait is explicit (vm_wait); the compiler's own, for the code registers, counts
//   only its loads and so waits somewhat longer than needed.
// MFMA t (0..3) of a step covers K offsets 32 q + 8 t .. + 7 in lane group q for both operands.
// Out-of-range W rows: their codes are read from the last row and their block scales read 0
// (buffer extent), as do X rows past M; steps past a wave's last one reload that step (unused).
template <int MB, int D, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void k_gemm_w4a16(const uint16_t *__restrict__ X,
                                                       const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ bscale,
                                                       const float *__restrict__ tscale,
                                                       int64_t M, int64_t N, int64_t K,
                                                       void *__restrict__ Y)
{
    constexpr int XBYTES = MB * 4 * 64 * 16;  // X per wave and step
    constexpr int SLOT = XBYTES + 2 * 64 * 4; // + the 64 rows' 8 scale bytes
    constexpr int NLOAD = 4 + 2 + 4 * MB;     // loads per wave and step: codes, scales, X
    static_assert((D - 1) * NLOAD < 64, "vmcnt range");
    static_assert(4 * D * SLOT >= 4 * 4 * MB * 64 * 16, "the partials fit in the ring");
    __shared__ __attribute__((aligned(16))) uint8_t xring[4][D][SLOT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lq = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 64, m0 = (int64_t)blockIdx.y * (16 * MB);
    const int64_t steps = K / 128;
    const int64_t mine = steps > wave ? (steps - wave + 3) / 4 : 0;

    const uint8_t *wrow[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int64_t n = n0 + 16 * nb + ln;
        wrow[nb] = codes + (n < N ? n : N - 1) * (K / 2) + 16 * lq;
    }
    // the workgroup's block scales, rows n0 .. N - 1 (rows past N read zeros)
    const int64_t kb = K / 16;
    const v4i_sgpr rs = make_rsrc_sgpr(bscale + n0 * kb, (uint32_t)((N - n0 < 64 ? N - n0 : 64) * kb));
    const uint32_t soff = (uint32_t)(lane * kb);   // + 8 s + 4 h
    // X through a buffer descriptor over rows m0 .. M - 1: rows past M read zeros
    const v4i_sgpr rx = make_rsrc_sgpr(X + m0 * K, (uint32_t)((M - m0) * K * 2));
    // this lane's chunk of a 4-row x 256-byte X load: row 4 p + lane / 16 of the block, chunk
    // (lane % 16) ^ row (the LDS slot it lands in is lane % 16)
    const int xr = lane >> 4, xs_slot = lane & 15;
    auto x_off = [&](int mb, int p, int64_t s) -> uint32_t {
        const int r = 16 * mb + 4 * p + xr;
        const int c = xs_slot ^ (r & 15);
        return (uint32_t)(((int64_t)r * K + 128 * s + 8 * c) * 2);
    };
    const uint32_t ring = lds_addr_of(&xring[wave][0][0]);

    auto step_of = [&](int64_t i) { return wave + 4 * (i < mine ? i : mine - 1); };
    auto refill = [&](int64_t i, int slot, uint4 (&c)[4]) {
        const int64_t s = step_of(i);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            c[nb] = *reinterpret_cast<const uint4 *>(wrow[nb] + 64 * s);
        // the slot's previous contents are read (their LDS reads returned) before refilling
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            dma4(rs, ring + (uint32_t)(slot * SLOT + XBYTES + 256 * h), soff + (uint32_t)(8 * s + 4 * h));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int p = 0; p < 4; ++p)
                dma16(rx, ring + (uint32_t)(slot * SLOT + (mb * 4 + p) * 1024), x_off(mb, p, s));
    };

    v4f acc[4][MB];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};

    // Every load is issued on every path (clamped past the end), so the number of loads issued
    // after a step's X is always (D - 1) NLOAD when the step waits for it.
    if (mine > 0) {
        uint4 cw[D][4];
#pragma unroll
        for (int j = 0; j < D; ++j)
            refill(j, j, cw[j]);
        for (int64_t i0 = 0; i0 < mine; i0 += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const int64_t i = i0 + j;
                if (i < mine) {
                    vm_wait<(D - 1) * NLOAD>();
                    const uint8_t *xs = &xring[wave][j][0];
                    float sc[4][2];
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) {
                        // row 16 nb + l % 16, scale bytes 2 q, 2 q + 1 of the step
                        const uint32_t b2 = *reinterpret_cast<const uint16_t *>(
                            xs + XBYTES + 256 * (lq >> 1) + 4 * (16 * nb + ln) + 2 * (lq & 1));
                        sc[nb][0] = __builtin_amdgcn_cvt_f32_fp8((int)(b2 & 0xFFu), 0);
                        sc[nb][1] = __builtin_amdgcn_cvt_f32_fp8((int)(b2 >> 8), 0);
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        v8bf wf[4];
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb) {
                            const uint32_t c8 = t == 0 ? cw[j][nb].x : t == 1 ? cw[j][nb].y
                                              : t == 2 ? cw[j][nb].z : cw[j][nb].w;
                            wf[nb] = dequant8(c8, sc[nb][t >> 1]);
                        }
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            // row 16 mb + l % 16, K offsets 32 q + 8 t .. + 7 = chunk 4 q + t
                            const v8bf xf = *reinterpret_cast<const v8bf *>(
                                xs + (16 * mb + ln) * 256 + (((4 * lq + t) ^ ln) << 4));
#pragma unroll
                            for (int nb = 0; nb < 4; ++nb)
                                acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    wf[nb], xf, acc[nb][mb], 0, 0, 0);
                        }
                    }
                }
                refill(i + D, j, cw[j]);
            }
        }
    }
    vm_wait<0>();   // the ring's last refills land before the ring is reused below
    __syncthreads();

    v4f(*red)[4 * MB][64] = reinterpret_cast<v4f(*)[4 * MB][64]>(&xring[0][0][0]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            red[wave][nb * MB + mb][lane] = acc[nb][mb];
    __syncthreads();

    // lane l of block (nb, mb) holds Y[m = m0 + 16 mb + l % 16][n = n0 + 16 nb + 4 (l / 16) + r]
    const float t = *tscale;
    for (int idx = tid; idx < 4 * MB * 64; idx += 256) {
        const int blk = idx >> 6, l = idx & 63;
        const v4f p = red[0][blk][l] + red[1][blk][l] + red[2][blk][l] + red[3][blk][l];
        const int nb = blk / MB, mb = blk % MB;
        const int64_t m = m0 + 16 * mb + (l & 15);
        const int64_t n = n0 + 16 * nb + 4 * (l >> 4);
        if (m >= M)
            continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = p[r] * t;
        const bool vec_ok = (N & 3) == 0 && n + 3 < N;
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

template <int MB, int D>
void launch_w4a16_cfg(bool out_bf16, const uint16_t *X, const uint8_t *codes,
                      const uint8_t *bscale, const float *tscale, int64_t M, int64_t N,
                      int64_t K, void *Y, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 16 * MB - 1) / (16 * MB)));
    if (out_bf16)
        k_gemm_w4a16<MB, D, true><<<grid, 256, 0, stream>>>(X, codes, bscale, tscale, M, N, K, Y);
    else
        k_gemm_w4a16<MB, D, false><<<grid, 256, 0, stream>>>(X, codes, bscale, tscale, M, N, K, Y);
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
    if (M <= 16)
        launch_w4a16_cfg<1, QR_W4_D1>(out_bf16, X, codes, bscale, tscale, M, N, K, Y, stream);
    else if (M <= QR_W4_M2)
        launch_w4a16_cfg<2, QR_W4_D2>(out_bf16, X, codes, bscale, tscale, M, N, K, Y, stream);
    else
        launch_w4a16_cfg<4, QR_W4_D4>(out_bf16, X, codes, bscale, tscale, M, N, K, Y, stream);
    return hipGetLastError();
}

}  // namespace qr
