// Quantizer kernels for gfx950: 1x128 row groups, 128x1 column groups (stored transposed),
// 128x128 weight blocks (with an optional transposed copy), and the UAQ fold.
//
// Granularity follows the Jet-RL notes (arXiv 2601.14243v1), section on the fine-grained GEMM
// quantization scheme: activations and gradients per 1x128 group, weights per 128x128 block,
// WGrad's second operand per 128x1 group with the two WGrad quantizations fused into one
// read.  The UAQ fold follows the QuRL notes (ICLR 2026), key design 1.
//
// One kernel template covers every quantizer.  A workgroup of 256 threads owns a 128x128
// bf16 tile (32 KB).  Thread t holds rows 8*(t/16)..+7 and columns 8*(t%16)..+7 of the tile
// as eight 16-byte loads, so each load instruction of a wave reads four full 256-byte row
// segments.  Group maxima are reduced in registers (DPP within a 16-lane row for row groups,
// lane shuffles plus LDS across waves for column groups and blocks); the 128 row scales and
// 128 column scales of a tile are then computed once each by one thread and shared through
// LDS, so the two divisions per group are not repeated by every lane.  Codes leave as 8-byte
// stores: in the input layout for row groups and blocks, and as 8 consecutive rows of one
// column for the transposed layouts (the column's group is contiguous there).
#include "qr_device.h"
#include "qr_internal.h"

namespace qr {

namespace {

constexpr int kTile = 128;

__device__ __forceinline__ uint32_t absmax8(const uint4 &v)
{
    return umax(umax(absmax2(v.x), absmax2(v.y)), umax(absmax2(v.z), absmax2(v.w)));
}

__device__ __forceinline__ uint32_t half_bits(const uint4 &v, int i)
{
    uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return ((i & 1) ? (w >> 16) : w) & 0x7FFFu;
}

__device__ __forceinline__ Scale scale_from(float s, float r)
{
    Scale sc;
    sc.s = s;
    sc.r = r;
    sc.slow = !(s >= 0x1p-100f);
    return sc;
}

// 8x8 byte transpose: in[j] holds row j (byte i = column i); out[i] holds column i
// (byte j = row j).  Four 4x4 transposes of v_perm_b32 each.
__device__ __forceinline__ void transpose4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                             uint32_t &y0, uint32_t &y1, uint32_t &y2,
                                             uint32_t &y3)
{
    uint32_t t0 = __builtin_amdgcn_perm(x1, x0, 0x06020400u);  // a0 b0 a2 b2
    uint32_t t1 = __builtin_amdgcn_perm(x1, x0, 0x07030501u);  // a1 b1 a3 b3
    uint32_t u0 = __builtin_amdgcn_perm(x3, x2, 0x06020400u);  // c0 d0 c2 d2
    uint32_t u1 = __builtin_amdgcn_perm(x3, x2, 0x07030501u);  // c1 d1 c3 d3
    y0 = __builtin_amdgcn_perm(u0, t0, 0x05040100u);           // a0 b0 c0 d0
    y2 = __builtin_amdgcn_perm(u0, t0, 0x07060302u);           // a2 b2 c2 d2
    y1 = __builtin_amdgcn_perm(u1, t1, 0x05040100u);           // a1 b1 c1 d1
    y3 = __builtin_amdgcn_perm(u1, t1, 0x07060302u);           // a3 b3 c3 d3
}

__device__ __forceinline__ void transpose8x8(const uint2 in[8], uint2 out[8])
{
    transpose4x4(in[0].x, in[1].x, in[2].x, in[3].x, out[0].x, out[1].x, out[2].x, out[3].x);
    transpose4x4(in[4].x, in[5].x, in[6].x, in[7].x, out[0].y, out[1].y, out[2].y, out[3].y);
    transpose4x4(in[0].y, in[1].y, in[2].y, in[3].y, out[4].x, out[5].x, out[6].x, out[7].x);
    transpose4x4(in[4].y, in[5].y, in[6].y, in[7].y, out[4].y, out[5].y, out[6].y, out[7].y);
}

template <int MODE>
__global__ __launch_bounds__(256) void k_quant_tile(const uint16_t *__restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ldx,
                                                    uint8_t *__restrict__ q,
                                                    float *__restrict__ s,
                                                    uint8_t *__restrict__ qT,
                                                    float *__restrict__ sT)
{
    constexpr bool ROW = (MODE & QMODE_ROW) != 0;
    constexpr bool COL = (MODE & QMODE_COL) != 0;
    constexpr bool BLK = (MODE & QMODE_BLK) != 0;
    constexpr bool BLKT = (MODE & QMODE_BLKT) != 0;
    constexpr bool ANYBLK = BLK || BLKT;

    __shared__ uint32_t red_col[4][kTile];
    __shared__ uint32_t red_row[kTile];
    __shared__ uint32_t red_blk[4];
    __shared__ float row_s[kTile], row_r[kTile], col_s[kTile], col_r[kTile];
    __shared__ float blk_sr[2];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int oq = t >> 4;   // row octet within the tile
    const int oc = t & 15;   // column octet within the tile
    const int64_t bi = blockIdx.y, bj = blockIdx.x;
    const int64_t r0 = bi * kTile, c0 = bj * kTile;
    const int64_t col = c0 + 8 * oc;
    const int64_t ngr = (rows + kTile - 1) / kTile, ngc = (cols + kTile - 1) / kTile;
    const bool colok = col < cols;

    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t r = r0 + 8 * oq + j;
        v[j] = make_uint4(0, 0, 0, 0);
        if (colok && r < rows)
            v[j] = *reinterpret_cast<const uint4 *>(x + r * ldx + col);
    }

    // ---- maxima
    if (ROW) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t m = row16_max(absmax8(v[j]));
            if (oc == 0)
                red_row[8 * oq + j] = m;
        }
    }
    if (COL) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m = umax(m, half_bits(v[j], i));
            m = umax(m, (uint32_t)__shfl_xor((int)m, 16));
            m = umax(m, (uint32_t)__shfl_xor((int)m, 32));
            if (lane < 16)
                red_col[wave][8 * oc + i] = m;
        }
    }
    if (ANYBLK) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            m = umax(m, absmax8(v[j]));
        m = row16_max(m);
        m = umax(m, (uint32_t)__shfl_xor((int)m, 16));
        m = umax(m, (uint32_t)__shfl_xor((int)m, 32));
        if (lane == 0)
            red_blk[wave] = m;
    }
    __syncthreads();

    // ---- scales: one thread per row, per column, per block
    if (ROW && t < kTile) {
        Scale sc = make_scale(red_row[t]);
        row_s[t] = sc.s;
        row_r[t] = sc.r;
        if (r0 + t < rows)
            s[(r0 + t) * ngc + bj] = sc.s;
    }
    if (COL && (ROW ? t >= kTile : t < kTile)) {
        const int c = ROW ? t - kTile : t;
        uint32_t m = umax(umax(red_col[0][c], red_col[1][c]), umax(red_col[2][c], red_col[3][c]));
        Scale sc = make_scale(m);
        col_s[c] = sc.s;
        col_r[c] = sc.r;
        if (c0 + c < cols)
            sT[(c0 + c) * ngr + bi] = sc.s;
    }
    if (ANYBLK && t == 0) {
        uint32_t m = umax(umax(red_blk[0], red_blk[1]), umax(red_blk[2], red_blk[3]));
        Scale sc = make_scale(m);
        blk_sr[0] = sc.s;
        blk_sr[1] = sc.r;
        if (BLK)
            s[bi * ngc + bj] = sc.s;
        if (BLKT)
            sT[bj * ngr + bi] = sc.s;
    }
    __syncthreads();

    // ---- codes
    if (ROW) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int rr = 8 * oq + j;
            const int64_t r = r0 + rr;
            uint2 c8 = encode8(v[j], scale_from(row_s[rr], row_r[rr]));
            if (colok && r < rows)
                *reinterpret_cast<uint2 *>(q + r * cols + col) = c8;
        }
    }
    if (ANYBLK) {
        const Scale sc = scale_from(blk_sr[0], blk_sr[1]);
        uint2 c8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            c8[j] = encode8(v[j], sc);
        if (BLK) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t r = r0 + 8 * oq + j;
                if (colok && r < rows)
                    *reinterpret_cast<uint2 *>(q + r * cols + col) = c8[j];
            }
        }
        if (BLKT) {
            uint2 ct[8];
            transpose8x8(c8, ct);
            const int64_t r = r0 + 8 * oq;   // rows % 8 == 0: the octet is all in or all out
            if (colok && r < rows) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint2 *>(qT + (col + i) * rows + r) = ct[i];
            }
        }
    }
    if (COL) {
        const int64_t r = r0 + 8 * oq;       // rows % 8 == 0: the octet is all in or all out
        const bool ok = colok && r < rows;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 8 * oc + i;
            const Scale sc = scale_from(col_s[c], col_r[c]);
            uint2 c8;
            c8.x = e4m3x4(quot(bf16_elem(v[0], i), sc), quot(bf16_elem(v[1], i), sc),
                          quot(bf16_elem(v[2], i), sc), quot(bf16_elem(v[3], i), sc));
            c8.y = e4m3x4(quot(bf16_elem(v[4], i), sc), quot(bf16_elem(v[5], i), sc),
                          quot(bf16_elem(v[6], i), sc), quot(bf16_elem(v[7], i), sc));
            if (ok)
                *reinterpret_cast<uint2 *>(qT + (col + i) * rows + r) = c8;
        }
    }
}

// ---------------------------------------------------------------- UAQ fold

// RN_bf16(w / s): the quotient is formed in binary64 (correctly rounded) and rounded to bf16
// directly from there.  When w / s is not a bf16 midpoint it lies at least ~2^-33 (relative)
// from every midpoint (w has 8 significant bits, s 24), far more than binary64's rounding
// error, so this equals rounding the exact quotient once.  (Rounding through binary32 first
// would not: binary32's 2^-24 step can land exactly on a midpoint.)
__device__ __forceinline__ uint16_t fold1(uint32_t wbits, float s)
{
    const float wv = __uint_as_float(wbits << 16);
    const double d = (double)wv / (double)s;
    const double a = fabs(d);
    double rv = 0.0;
    if (a != 0.0) {
        int e = ilogb(a);
        if (e < -126)
            e = -126;                                   // bf16 subnormal spacing 2^-133
        rv = ldexp(rint(ldexp(a, 7 - e)), e - 7);       // 8 significant bits, ties to even
    }
    const uint32_t fb = __float_as_uint((float)rv);    // exact (or overflow to inf)
    return (uint16_t)((fb >> 16) | (wbits & 0x8000u));
}

__global__ __launch_bounds__(256) void k_uaq_fold(const uint16_t *w, int64_t n, int64_t k,
                                                  int64_t ldw, const float *__restrict__ s,
                                                  uint16_t *out, int64_t ldo, float *gain)
{
    const int64_t chunks_per_row = k / 8;
    const int64_t total = n * chunks_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
        const int64_t row = c / chunks_per_row, kc = (c - row * chunks_per_row) * 8;
        const uint4 v = *reinterpret_cast<const uint4 *>(w + row * ldw + kc);
        const float4 s0 = *reinterpret_cast<const float4 *>(s + kc);
        const float4 s1 = *reinterpret_cast<const float4 *>(s + kc + 4);
        uint4 o;
        o.x = fold1(v.x & 0xFFFFu, s0.x) | ((uint32_t)fold1(v.x >> 16, s0.y) << 16);
        o.y = fold1(v.y & 0xFFFFu, s0.z) | ((uint32_t)fold1(v.y >> 16, s0.w) << 16);
        o.z = fold1(v.z & 0xFFFFu, s1.x) | ((uint32_t)fold1(v.z >> 16, s1.y) << 16);
        o.w = fold1(v.w & 0xFFFFu, s1.z) | ((uint32_t)fold1(v.w >> 16, s1.w) << 16);
        *reinterpret_cast<uint4 *>(out + row * ldo + kc) = o;
    }
    if (gain) {
        for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < k; c += stride)
            gain[c] = gain[c] * s[c];
    }
}

}  // namespace

hipError_t launch_quant_tile(int mode, const uint16_t *x, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t *q, float *s, uint8_t *qT, float *sT,
                             hipStream_t stream)
{
    const int64_t ngr = (rows + kTile - 1) / kTile, ngc = (cols + kTile - 1) / kTile;
    if (ngr == 0 || ngc == 0)
        return hipSuccess;
    dim3 grid((unsigned)ngc, (unsigned)ngr);
    switch (mode) {
    case QMODE_ROW:
        k_quant_tile<QMODE_ROW><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s, qT, sT);
        break;
    case QMODE_COL:
        k_quant_tile<QMODE_COL><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s, qT, sT);
        break;
    case QMODE_ROW | QMODE_COL:
        k_quant_tile<QMODE_ROW | QMODE_COL><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s,
                                                                      qT, sT);
        break;
    case QMODE_BLK:
        k_quant_tile<QMODE_BLK><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s, qT, sT);
        break;
    case QMODE_BLK | QMODE_BLKT:
        k_quant_tile<QMODE_BLK | QMODE_BLKT><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s,
                                                                       qT, sT);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_uaq_fold(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                           const float *s, uint16_t *w_out, int64_t ld_out, float *gain,
                           hipStream_t stream)
{
    const int64_t total = n * (k / 8);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 16384)
        blocks = 16384;
    if (blocks < 1)
        blocks = 1;
    k_uaq_fold<<<(unsigned)blocks, 256, 0, stream>>>(w, n, k, ld_w, s, w_out, ld_out, gain);
    return hipGetLastError();
}

}  // namespace qr
