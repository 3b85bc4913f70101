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
#include <type_traits>

#include "qr_device.h"
#include "qr_internal.h"

namespace qr {

namespace {

constexpr int kTile = 128;
#ifndef QR_QUANT_WG_PER_CU
#define QR_QUANT_WG_PER_CU 8
#endif
constexpr int kQuantWgPerCu = QR_QUANT_WG_PER_CU;   // resident workgroups per CU in the persistent grid
#ifndef QR_SMALL_ROWS
#define QR_SMALL_ROWS 256
#endif
constexpr int64_t kSmallRows = QR_SMALL_ROWS;   // row-group pass: up to this many rows, one wave per row slice

__device__ __forceinline__ uint32_t absmax8(const uint4 &v)
{
    return umax(umax(absmax2(v.x), absmax2(v.y)), umax(absmax2(v.z), absmax2(v.w)));
}

__device__ __forceinline__ uint32_t half_bits(const uint4 &v, int i)
{
    uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return ((i & 1) ? (w >> 16) : w) & 0x7FFFu;
}

__device__ __forceinline__ Scale unpack_scale(const float4 &p)
{
    Scale sc;
    sc.s = 0.0f;   // not needed by the encoder
    sc.sq = p.x;
    sc.r = p.y;
    sc.m = p.z;
    return sc;
}

__device__ __forceinline__ float4 pack_scale(const Scale &sc)
{
    return make_float4(sc.sq, sc.r, sc.m, 0.0f);
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

// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not for its global
// loads or stores.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr int kBufFlags = 0x00020000;     // raw buffer, range-checked per lane
constexpr uint32_t kOutOfRange = 0x80000000u;

// ---------------------------------------------------------------- UAQ fold

// RN_bf16(w / s), general case: the quotient is formed in binary64 (correctly rounded) and
// rounded to bf16 directly from there.  When w / s is not a bf16 midpoint it lies at least
// ~2^-33 (relative) from every midpoint (w has 8 significant bits, s 24), far more than
// binary64's rounding error, so this equals rounding the exact quotient once.  (Rounding
// through binary32 first would not: binary32's 2^-24 step can land exactly on a midpoint.)
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

// RN_bf16(w / s) for s > 0 with r = RN32(1 / s); `col_ok` says 2^-120 <= s < 2^121.
// z = |w| / s is bracketed without division: q = RN32(|w| * r) is within (2u + u^2) z of z
// (u = 2^-24: one rounding in r, one in the product), i.e. within 2.01 binary32 ulps of q.
// Let lo be q truncated to bf16 and hi = lo + one bf16 ulp.  Then z lies between the bf16
// midpoint below lo and the one above hi, so it rounds to lo or hi, and only its side of
// their midpoint m = lo + ulp / 2 is left to decide.  That is the sign of |w| - m * s, taken
// exactly from one FMA: |w| and m * s are multiples of 2^(E_w - 32) or coarser, so with
// |w| >= 2^-90 a non-zero difference is at least 2^-122 and its rounding keeps its sign; zero
// would be the tie (even neighbour).  `slow` flags the elements outside those ranges (tiny or
// huge quotients or weights, s out of range, non-finite w), which take the binary64 route;
// zero weights give the signed zero directly.
__device__ __forceinline__ uint32_t fold_fast(uint32_t wbits, float s, float r, bool col_ok,
                                              uint32_t &slow)
{
    const float a = __uint_as_float((wbits & 0x7FFFu) << 16);
    const uint32_t qb = __float_as_uint(a * r);
    const uint32_t ew = (wbits >> 7) & 0xFFu, eq = qb >> 23;
    const uint32_t lo = qb & 0xFFFF0000u;
    const float d = fmaf(-__uint_as_float(lo | 0x8000u), s, a);
    const uint32_t up = d > 0.0f ? 1u : (d == 0.0f ? (lo >> 16) & 1u : 0u);
    const bool zero = (wbits & 0x7FFFu) == 0;            // +-0 / s = +-0 for s > 0
    const bool ok = col_ok && ew >= 37u && eq - 27u <= 220u;
    slow = (ok || zero) ? 0u : 1u;
    return zero ? wbits : (((lo >> 16) + up) | (wbits & 0x8000u));
}

// The fold's per-lane constants for 8 adjacent columns: s, r = RN32(1 / s) (correctly
// rounded) and whether s lies in the fast route's range.
struct Fold8 {
    float s[8], r[8];
    bool ok[8];
};

__device__ __forceinline__ void fold8_setup(const float *__restrict__ s, int64_t c, Fold8 &f)
{
    const float4 s0 = *reinterpret_cast<const float4 *>(s + c);
    const float4 s1 = *reinterpret_cast<const float4 *>(s + c + 4);
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        f.s[j] = sv[j];
        f.r[j] = __fdiv_rn(1.0f, sv[j]);
        f.ok[j] = (__float_as_uint(sv[j]) >> 23) - 7u <= 240u;   // 2^-120 <= s < 2^121
    }
}

// RN_bf16(w / s) of 8 adjacent bf16 weights (one 16-byte chunk); the binary64 route only for
// chunks that hold an element outside the fast route's ranges.
__device__ __forceinline__ uint4 fold8(const uint4 &v, const Fold8 &f)
{
    const uint32_t wb[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                            v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
    uint32_t res[8], sl[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        res[j] = fold_fast(wb[j], f.s[j], f.r[j], f.ok[j], sl[j]);
    if (sl[0] | sl[1] | sl[2] | sl[3] | sl[4] | sl[5] | sl[6] | sl[7]) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (sl[j])
                res[j] = fold1(wb[j], f.s[j]);
    }
    return make_uint4(res[0] | (res[1] << 16), res[2] | (res[3] << 16),
                      res[4] | (res[5] << 16), res[6] | (res[7] << 16));
}

__device__ __forceinline__ float sumsq8(const uint4 &v, float ss)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = bf16_elem(v, i);
        ss = __builtin_fmaf(x, x, ss);   // x * x is exact in binary32 (8-bit significands)
    }
    return ss;
}

// y = RN_bf16((h * inv) * gain) for 8 consecutive elements.  The binary32 products are
// rounded to bf16 in pairs by the packed conversion, round to nearest even (finite values,
// subnormals kept).
__device__ __forceinline__ uint4 rms_apply(const uint4 &v, float inv, const float4 &g0,
                                           const float4 &g1)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2_t t = {bf16_elem(v, 2 * i) * inv * g[2 * i],
                           bf16_elem(v, 2 * i + 1) * inv * g[2 * i + 1]};
        o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(t, bf16x2_t));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// The norm ahead of an activation quantization: the tile's bf16 values h are replaced by
// y = RN_bf16((h * inv[r]) * gain[c]) (the row statistics inv come from k_rms_inv) before the
// maxima, and written to y if asked for.
struct NormArgs {
    const float *inv = nullptr;    // [rows]
    const float *gain = nullptr;   // [cols]
    uint16_t *y = nullptr;         // [rows, cols] dense, or nullptr
};

// The fold ahead of a 128x128 weight quantization: the tile's bf16 values are replaced by
// RN_bf16(w / s[c]) before the block maxima, written to out, and the gain is scaled by s once.
struct FoldArgs {
    const float *s = nullptr;   // [cols]
    uint16_t *out = nullptr;    // [rows, cols], leading dimension ldo (may equal the input)
    int64_t ldo = 0;
    float *gain = nullptr;      // [cols] or nullptr
};

// The tile's eight 16-byte loads per thread as range-checked buffer loads: a row past `rows`
// lies past the descriptor's extent and a column octet past `cols` takes an offset outside it,
// so both read zeros without a branch.
__device__ __forceinline__ void load_tile(const uint16_t *__restrict__ x, int64_t rows,
                                          int64_t ldx, int64_t r0, int64_t col, bool colok,
                                          int oq, uint4 v[8])
{
    int64_t extent = (rows - r0) * ldx * 2;
    if (extent > 0x7FFFFFF0)
        extent = 0x7FFFFFF0;
    if (extent < 0)
        extent = 0;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + r0 * ldx), 0, (int)extent, kBufFlags);
    const uint32_t base = (uint32_t)(8 * oq * ldx + col) * 2u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t off = colok ? base + (uint32_t)(j * ldx * 2) : kOutOfRange;
        v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
    }
}

// The workgroup handles tiles first, first + stride, ... of x (row-major over the tile grid).
// Every thread of the workgroup calls it.
template <int MODE>
__device__ __forceinline__ void quant_tiles(const uint16_t *x, int64_t rows,
                                            int64_t cols, int64_t ldx, uint8_t *__restrict__ q,
                                            float *__restrict__ s, uint8_t *__restrict__ qT,
                                            float *__restrict__ sT, int64_t first, int64_t stride,
                                            int64_t pend, const FoldArgs fa = FoldArgs{},
                                            const NormArgs na = NormArgs{})
{
    constexpr bool ROW = (MODE & QMODE_ROW) != 0;
    constexpr bool COL = (MODE & QMODE_COL) != 0;
    constexpr bool BLK = (MODE & QMODE_BLK) != 0;
    constexpr bool BLKT = (MODE & QMODE_BLKT) != 0;
    constexpr bool FOLD = (MODE & QMODE_FOLD) != 0;
    constexpr bool NORM = (MODE & QMODE_NORM) != 0;
    constexpr bool ANYBLK = BLK || BLKT;

    __shared__ uint32_t red_col[4][kTile];
    __shared__ uint32_t red_row[kTile];
    __shared__ uint32_t red_blk[4];
    __shared__ float4 row_sc[kTile], col_sc[kTile];
    __shared__ float4 blk_sc;
    __shared__ uint32_t tiny_flag[2];   // per iteration parity: some group of the tile is tiny
    // Transposed codes of the tile, staged so that they leave as whole 128-byte column
    // segments: row c holds column c0 + c (its 128 tile rows, one byte each); its 16-byte
    // chunk k (tile rows 16 k .. 16 k + 15) sits in slot k ^ ((c / 8) % 8).
    constexpr bool STAGE_T = COL || BLKT;
    __shared__ __attribute__((aligned(16))) uint8_t tcodes[STAGE_T ? kTile * kTile : 16];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int oq = t >> 4;   // row octet within the tile
    const int oc = t & 15;   // column octet within the tile
    const int64_t ngr = (rows + kTile - 1) / kTile, ngc = (cols + kTile - 1) / kTile;

    auto process = [&](int64_t bi, int64_t bj, int par, uint4 (&v)[8]) {
        const int64_t r0 = bi * kTile, c0 = bj * kTile;
        const int64_t col = c0 + 8 * oc;
        const bool colok = col < cols;
        // 8 codes of tile column c, tile rows 8 oq .. 8 oq + 7, into the staging tile
        auto stage_t = [&](int c, uint2 codes8) {
            *reinterpret_cast<uint2 *>(tcodes + c * kTile + (((oq >> 1) ^ ((c >> 3) & 7)) << 4) +
                                       8 * (oq & 1)) = codes8;
        };

        // ---- maxima
        if (t == 0)
            tiny_flag[par] = 0;   // last read two iterations ago, before two barriers
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
        lds_barrier();

        // ---- scales: one thread per row, per column, per block
        if (ROW && t < kTile) {
            const Scale sc = make_scale(red_row[t]);
            row_sc[t] = pack_scale(sc);
            if (tiny_scale(sc))
                tiny_flag[par] = 1;
            if (r0 + t < rows)
                s[(r0 + t) * ngc + bj] = sc.s;
        }
        if (COL && (ROW ? t >= kTile : t < kTile)) {
            const int c = ROW ? t - kTile : t;
            const uint32_t m = umax(umax(red_col[0][c], red_col[1][c]),
                                    umax(red_col[2][c], red_col[3][c]));
            const Scale sc = make_scale(m);
            col_sc[c] = pack_scale(sc);
            if (tiny_scale(sc))
                tiny_flag[par] = 1;
            if (c0 + c < cols)
                sT[(c0 + c) * ngr + bi] = sc.s;
        }
        if (ANYBLK && t == 0) {
            const uint32_t m = umax(umax(red_blk[0], red_blk[1]), umax(red_blk[2], red_blk[3]));
            const Scale sc = make_scale(m);
            blk_sc = pack_scale(sc);
            if (tiny_scale(sc))
                tiny_flag[par] = 1;
            if (BLK)
                s[bi * ngc + bj] = sc.s;
            if (BLKT)
                sT[bj * ngr + bi] = sc.s;
        }
        lds_barrier();

        // ---- codes (the lifted quotient only for tiles that hold a tiny scale)
        auto encode = [&](auto lift_tag) {
            constexpr bool LIFT = decltype(lift_tag)::value;
            if (ROW) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int rr = 8 * oq + j;
                    const int64_t r = r0 + rr;
                    const uint2 c8 = encode8<LIFT>(v[j], unpack_scale(row_sc[rr]));
                    if (colok && r < rows)
                        *reinterpret_cast<uint2 *>(q + r * cols + col) = c8;
                }
            }
            if (ANYBLK) {
                const Scale sc = unpack_scale(blk_sc);
                uint2 c8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    c8[j] = encode8<LIFT>(v[j], sc);
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
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        stage_t(8 * oc + i, ct[i]);
                }
            }
            if (COL) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const Scale sc = unpack_scale(col_sc[8 * oc + i]);
                    uint2 c8;
                    c8.x = e4m3x4(quot_t<LIFT>(bf16_elem(v[0], i), sc),
                                  quot_t<LIFT>(bf16_elem(v[1], i), sc),
                                  quot_t<LIFT>(bf16_elem(v[2], i), sc),
                                  quot_t<LIFT>(bf16_elem(v[3], i), sc));
                    c8.y = e4m3x4(quot_t<LIFT>(bf16_elem(v[4], i), sc),
                                  quot_t<LIFT>(bf16_elem(v[5], i), sc),
                                  quot_t<LIFT>(bf16_elem(v[6], i), sc),
                                  quot_t<LIFT>(bf16_elem(v[7], i), sc));
                    stage_t(8 * oc + i, c8);
                }
            }
        };
        if (__builtin_amdgcn_readfirstlane(tiny_flag[par]))
            encode(std::true_type{});
        else
            encode(std::false_type{});

        // ---- transposed codes leave the staging tile as whole column segments: a wave
        // stores 8 columns x 128 bytes per instruction.  (The next tile writes the staging
        // tile only after two more barriers, so one buffer is enough.)
        if (STAGE_T) {
            lds_barrier();
            const bool whole16 = (rows & 15) == 0;   // every column segment 16-byte aligned
#pragma unroll
            for (int p = 0; p < kTile * kTile / 16 / 256; ++p) {
                const int c = p * 32 + (t >> 3), ch = t & 7;
                const uint4 d = *reinterpret_cast<const uint4 *>(
                    tcodes + c * kTile + ((ch ^ ((c >> 3) & 7)) << 4));
                const int64_t cc = c0 + c, r = r0 + 16 * ch;   // rows % 8 == 0
                if (cc >= cols || r >= rows)
                    continue;
                uint8_t *dst = qT + cc * rows + r;
                if (whole16 && r + 16 <= rows) {
                    *reinterpret_cast<uint4 *>(dst) = d;
                } else {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(d.x, d.y);
                    if (r + 8 < rows)
                        *reinterpret_cast<uint2 *>(dst + 8) = make_uint2(d.z, d.w);
                }
            }
        }
    };

    // One tile at a time: load it, then reduce, encode and store it.  The load latency is
    // covered by the other workgroups resident on the CU, not by a second register buffer:
    // without one every mode needs at most 168 VGPRs, so 3 to 8 workgroups fit per CU.  (A
    // prefetch of the next tile into a second register set measured slower for every mode at
    // 8192x4096: rows 25.1 against 23.0 us, columns 25.5 against 23.2, dual 36.7 against
    // 33.6, weight blocks with the transposed copy 16.1 against 15.3.)
    // Tile (bi, bj) is walked incrementally (no 64-bit division in the loop); the walk visits
    // linear tile indices first, first + stride, ... below pend (at most the tile count).
    const int64_t dbi = stride / ngc, dbj = stride - dbi * ngc;
    int64_t pi = first, bi = first / ngc, bj = first - bi * ngc;
    int par = 0;
    while (pi < pend) {
        uint4 v[8];
        const int64_t c = bj * kTile + 8 * oc;
        load_tile(x, rows, ldx, bi * kTile, c, c < cols, oq, v);
        if (FOLD && c < cols) {
            // this thread's 8 columns of the tile's rows 8 oq .. 8 oq + 7 (only this thread
            // reads or writes them, so out may be the input itself)
            Fold8 f;
            fold8_setup(fa.s, c, f);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[j] = fold8(v[j], f);
                const int64_t r = bi * kTile + 8 * oq + j;
                if (r < rows)
                    *reinterpret_cast<uint4 *>(fa.out + r * fa.ldo + c) = v[j];
            }
            if (fa.gain && bi == 0 && oq == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    fa.gain[c + j] = fa.gain[c + j] * f.s[j];
            }
        }
        if (NORM && c < cols) {
            // this thread's 8 columns of the tile's rows 8 oq .. 8 oq + 7 (rows past the end
            // stay zero)
            const float4 g0 = *reinterpret_cast<const float4 *>(na.gain + c);
            const float4 g1 = *reinterpret_cast<const float4 *>(na.gain + c + 4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t r = bi * kTile + 8 * oq + j;
                if (r < rows) {
                    v[j] = rms_apply(v[j], na.inv[r], g0, g1);
                    if (na.y)
                        *reinterpret_cast<uint4 *>(na.y + r * cols + c) = v[j];
                }
            }
        }
        process(bi, bj, par, v);
        par ^= 1;
        pi += stride;
        bi += dbi;
        bj += dbj;
        if (bj >= ngc) {
            bj -= ngc;
            ++bi;
        }
    }
}

// Persistent: as many workgroups as fit on the CUs at once; workgroup b handles tiles
// first(b), first(b) + gridDim.x, ... (row-major over the tile grid), so at any time the grid
// works on one contiguous window of tiles.  first(b) = b, except for the row-group pass when
// the window holds whole row bands, 8 or more: ids are dealt round-robin to the 8 XCDs, and
// XCD x (ids b with b mod 8 = x) then takes whole row bands x, x + 8, ... of each window, so
// the 4-byte row-scale stores of a band (its tiles' scales share 128-byte lines) merge in one
// L2 before they are written back.  (The column pass keeps first(b) = b: with 128-column
// tiles and a row of tiles a multiple of 8 long, a column band already stays on one XCD.)
template <int MODE>
// At least 3 waves per SIMD (3 workgroups per CU): the register budget is 168 VGPRs, which
// every mode meets without spilling.
__global__ __launch_bounds__(256, 3) void k_quant_tile(const uint16_t *__restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ldx,
                                                    uint8_t *__restrict__ q,
                                                    float *__restrict__ s,
                                                    uint8_t *__restrict__ qT,
                                                    float *__restrict__ sT)
{
    const int64_t ngc = (cols + kTile - 1) / kTile;
    const int64_t nt = ((rows + kTile - 1) / kTile) * ngc;
    const int64_t G = gridDim.x;
    int64_t first = blockIdx.x;
    if (MODE == QMODE_ROW && (G & 7) == 0 && (G / 8) % ngc == 0) {
        const int64_t xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
        first = (xcd + 8 * (l / ngc)) * ngc + l % ngc;
    }
    quant_tiles<MODE>(x, rows, cols, ldx, q, s, qT, sT, first, G, nt);
}

// The UAQ fold and the 128x128 weight quantization in one pass (MODE = BLK | FOLD, plus BLKT
// for the transposed copy): each tile is folded in registers, written out, and quantized.
// x is not restrict-qualified here or in quant_tiles: in place, the folded values go back to
// x's own memory.
template <int MODE>
__global__ __launch_bounds__(256, 3) void k_fold_quant_w(const uint16_t *x,
                                                      int64_t rows, int64_t cols, int64_t ldx,
                                                      uint8_t *__restrict__ q,
                                                      float *__restrict__ s,
                                                      uint8_t *__restrict__ qT,
                                                      float *__restrict__ sT, FoldArgs fa)
{
    const int64_t ngc = (cols + kTile - 1) / kTile;
    const int64_t nt = ((rows + kTile - 1) / kTile) * ngc;
    quant_tiles<MODE>(x, rows, cols, ldx, q, s, qT, sT, blockIdx.x, gridDim.x, nt, fa);
}

// The norm and the activation quantization in one pass over h (MODE = ROW and/or COL, plus
// NORM): each tile is normalized in registers (and written to y if asked for), then quantized.
template <int MODE>
__global__ __launch_bounds__(256, 3) void k_norm_quant_tile(const uint16_t *__restrict__ h,
                                                         int64_t rows, int64_t cols, int64_t ldh,
                                                         uint8_t *__restrict__ q,
                                                         float *__restrict__ s,
                                                         uint8_t *__restrict__ qT,
                                                         float *__restrict__ sT, NormArgs na)
{
    const int64_t ngc = (cols + kTile - 1) / kTile;
    const int64_t nt = ((rows + kTile - 1) / kTile) * ngc;
    quant_tiles<MODE>(h, rows, cols, ldh, q, s, qT, sT, blockIdx.x, gridDim.x, nt, FoldArgs{},
                      na);
}

// A row's norm statistic inv = 1 / sqrt(mean(h^2) + eps), one wave per row, with the sum of
// squares in k_rmsnorm_quant's order (lane sums over the 512-column passes in pass order, then
// the same 64-lane butterfly), so the normalized values equal that kernel's.
__global__ __launch_bounds__(256) void k_rms_inv(const uint16_t *__restrict__ h, int64_t rows,
                                                 int64_t cols, int64_t ldh, float eps,
                                                 float *__restrict__ inv)
{
    const int lane = threadIdx.x & 63, sub = lane >> 4, li = lane & 15;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;   // the whole wave; no barrier follows
    const int64_t ngc = (cols + kTile - 1) / kTile, npass = (ngc + 3) / 4;
    const uint16_t *hr = h + row * ldh;
    float ss = 0.0f;
    for (int64_t p = 0; p < npass; ++p) {
        const int64_t c = (4 * p + sub) * kTile + 8 * li;
        const uint4 v = c < cols ? *reinterpret_cast<const uint4 *>(hr + c) : make_uint4(0, 0, 0, 0);
        ss = sumsq8(v, ss);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        ss += __shfl_xor(ss, o);
    if (lane == 0)
        inv[row] = 1.0f / sqrtf(ss / (float)cols + eps);
}

// A list of weights quantized in one persistent launch (a weight update re-quantizes every
// layer).  The tiles of all tensors form one round-robin sequence over the workgroups, so a
// small tensor does not leave most of the grid idle.  The table travels by value in the
// kernel arguments.
template <int MODE>
__global__ __launch_bounds__(256) void k_quant_w_batch(WeightTable tab)
{
    const int64_t G = gridDim.x;
    int64_t before = 0;   // tiles of the tensors already walked
    for (int i = 0; i < tab.count; ++i) {
        const WeightDesc &d = tab.d[i];
        int64_t first = ((int64_t)blockIdx.x - before) % G;
        if (first < 0)
            first += G;
        quant_tiles<MODE>(d.w, d.n, d.k, d.ld, d.q, d.s, d.qT, d.sT, first, G, d.tiles);
        before += d.tiles;
        __syncthreads();   // LDS of this tensor's last tile is read before the next one writes
    }
}

// 1x128 row groups of a few rows (decode activations): one wave per row and 512-column slice,
// lanes 16 t .. 16 t + 15 on group t of the slice (8 columns each), so a 64 x 4096 activation
// takes 512 waves instead of 32 half-empty 128-row tiles.  Same maxima, scales and encoder as
// the tile kernel's row mode (the lifted quotient only for groups with a tiny scale; for the
// others it is the same quotient).
__global__ __launch_bounds__(256) void k_quant_rows_small(const uint16_t *__restrict__ x,
                                                          int64_t rows, int64_t cols,
                                                          int64_t ldx, uint8_t *__restrict__ q,
                                                          float *__restrict__ s)
{
    const int lane = threadIdx.x & 63, sub = lane >> 4, li = lane & 15;
    const int64_t ngc = (cols + kTile - 1) / kTile, nslice = (ngc + 3) / 4;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t row = wid / nslice, sl = wid - row * nslice;
    if (row >= rows)
        return;   // the whole wave; no barrier follows
    const int64_t g = 4 * sl + sub, c = g * kTile + 8 * li;
    const bool ok = c < cols;   // cols % 8 == 0: an octet is all in or out
    const uint4 v = ok ? *reinterpret_cast<const uint4 *>(x + row * ldx + c) : make_uint4(0, 0, 0, 0);
    const Scale sc = make_scale(row16_max(absmax8(v)));   // all 64 lanes take part
    const uint2 c8 = tiny_scale(sc) ? encode8<true>(v, sc) : encode8<false>(v, sc);
    if (ok)
        *reinterpret_cast<uint2 *>(q + row * cols + c) = c8;
    if (li == 0 && g < ngc)
        s[row * ngc + g] = sc.s;
}

// ---------------------------------------------------------------- RMSNorm + 1x128 quantize

// The norm in front of a linear layer with its 1x128 quantization fused in: one wave per row.
// In pass p, lanes 16 t .. 16 t + 15 take 128-column group 4 p + t, 8 columns (16 bytes)
// each, so a pass reads 1 KB of the row and a group's max is a 16-lane DPP reduction.  The
// first phase sums h^2 (NP > 0: the row stays in registers, NP passes at most; NP == 0: the
// second phase reads it again); the second forms y = RN_bf16((h * inv) * gain) with
// inv = 1 / sqrt(sum / cols + eps) and encodes y exactly as the 1x128 quantizer does.
// FULL: cols is exactly NP passes (4096 columns for NP = 8), so no column checks; the gain
// octets of the next pass are loaded while the current one is encoded.
template <int NP, bool FULL>
__global__ __launch_bounds__(256) void k_rmsnorm_quant(const uint16_t *__restrict__ h,
                                                       int64_t rows, int64_t cols, int64_t ldh,
                                                       const float *__restrict__ gain, float eps,
                                                       uint16_t *__restrict__ y,
                                                       uint8_t *__restrict__ q,
                                                       float *__restrict__ s)
{
    static_assert(!FULL || NP > 0, "whole passes keep the row in registers");
    const int lane = threadIdx.x & 63, sub = lane >> 4, li = lane & 15;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;   // the whole wave; no barrier follows
    const int64_t ngc = (cols + kTile - 1) / kTile, npass = FULL ? NP : (ngc + 3) / 4;
    const uint16_t *hr = h + row * ldh;
    auto col_of = [&](int64_t p) { return (int)((4 * p + sub) * kTile + 8 * li); };
    auto in_row = [&](int64_t c) { return FULL || c < cols; };
    auto load = [&](int64_t p) -> uint4 {
        const int64_t c = col_of(p);   // cols % 8 == 0: an octet is all in or out
        return in_row(c) ? *reinterpret_cast<const uint4 *>(hr + c) : make_uint4(0, 0, 0, 0);
    };
    float ss = 0.0f;
    uint4 keep[NP > 0 ? NP : 1];
    if (NP > 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            keep[p] = p < npass ? load(p) : make_uint4(0, 0, 0, 0);
            ss = sumsq8(keep[p], ss);
        }
    } else {
        for (int64_t p = 0; p < npass; ++p)
            ss = sumsq8(load(p), ss);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        ss += __shfl_xor(ss, o);       // every lane ends with the same sum
    const float inv = 1.0f / sqrtf(ss / (float)cols + eps);

    // the gain octet of pass p; a column past the row reads octet 0 instead (values unused)
    auto gload = [&](int64_t p, float4 &g0, float4 &g1) {
        const int64_t c = in_row(col_of(p)) ? col_of(p) : 0;
        g0 = *reinterpret_cast<const float4 *>(gain + c);
        g1 = *reinterpret_cast<const float4 *>(gain + c + 4);
    };
    auto body = [&](int64_t p, const uint4 &v, const float4 &g0, const float4 &g1) {
        const int64_t c = col_of(p);
        const bool ok = in_row(c);
        uint4 yv = make_uint4(0, 0, 0, 0);
        if (ok) {
            yv = rms_apply(v, inv, g0, g1);
            if (y)
                *reinterpret_cast<uint4 *>(y + row * cols + c) = yv;
        }
        const Scale sc = make_scale(row16_max(absmax8(yv)));   // all 64 lanes take part
        const uint2 c8 = tiny_scale(sc) ? encode8<true>(yv, sc) : encode8<false>(yv, sc);
        if (ok)
            *reinterpret_cast<uint2 *>(q + row * cols + c) = c8;
        const int64_t g = 4 * p + sub;
        if (li == 0 && (FULL || g < ngc))
            s[row * ngc + g] = sc.s;
    };
    if (NP > 0) {
        float4 ga0, ga1, gb0, gb1;
        gload(0, ga0, ga1);
#pragma unroll
        for (int p = 0; p < NP; ++p)
            if (p < npass) {   // uniform across the wave
                if (p + 1 < NP && p + 1 < npass)
                    gload(p + 1, gb0, gb1);     // one pass ahead
                body(p, keep[p], ga0, ga1);
                ga0 = gb0;
                ga1 = gb1;
            }
    } else {
        for (int64_t p = 0; p < npass; ++p) {
            float4 g0, g1;
            gload(p, g0, g1);
            body(p, load(p), g0, g1);
        }
    }
}

// The same norm and quantize for few rows (decode batches): one workgroup of SW waves per row.
// Wave w takes the row's 512-column passes w, w + SW, ...; the waves' partial sums of squares
// meet in LDS and every wave adds them in wave order, so the sum (and y) does not depend on
// timing.  NP > 0: a wave keeps its NP passes in registers; NP == 0: it reads them twice.
template <int NP, int SW>
__global__ __launch_bounds__(64 * SW) void k_rmsnorm_quant_split(
    const uint16_t *__restrict__ h, int64_t rows, int64_t cols, int64_t ldh,
    const float *__restrict__ gain, float eps, uint16_t *__restrict__ y, uint8_t *__restrict__ q,
    float *__restrict__ s)
{
    __shared__ float part[SW];
    const int lane = threadIdx.x & 63, sub = lane >> 4, li = lane & 15;
    const int w = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;   // grid = rows: every wave of the workgroup has a row
    const int64_t ngc = (cols + kTile - 1) / kTile, npass = (ngc + 3) / 4;
    const uint16_t *hr = h + row * ldh;
    auto col_of = [&](int64_t p) { return (4 * p + sub) * kTile + 8 * li; };
    auto load = [&](int64_t p) -> uint4 {
        const int64_t c = col_of(p);   // cols % 8 == 0: an octet is all in or out
        return p < npass && c < cols ? *reinterpret_cast<const uint4 *>(hr + c)
                                     : make_uint4(0, 0, 0, 0);
    };
    float ss = 0.0f;
    uint4 keep[NP > 0 ? NP : 1];
    if (NP > 0) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            keep[j] = load(w + (int64_t)j * SW);
            ss = sumsq8(keep[j], ss);
        }
    } else {
        for (int64_t p = w; p < npass; p += SW)
            ss = sumsq8(load(p), ss);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        ss += __shfl_xor(ss, o);
    if (lane == 0)
        part[w] = ss;
    __syncthreads();
    float tot = part[0];
#pragma unroll
    for (int k = 1; k < SW; ++k)
        tot += part[k];
    const float inv = 1.0f / sqrtf(tot / (float)cols + eps);

    auto body = [&](int64_t p, const uint4 &v) {
        const int64_t c = col_of(p);
        const bool ok = p < npass && c < cols;
        uint4 yv = make_uint4(0, 0, 0, 0);
        if (ok) {
            const float4 g0 = *reinterpret_cast<const float4 *>(gain + c);
            const float4 g1 = *reinterpret_cast<const float4 *>(gain + c + 4);
            yv = rms_apply(v, inv, g0, g1);
            if (y)
                *reinterpret_cast<uint4 *>(y + row * cols + c) = yv;
        }
        const Scale sc = make_scale(row16_max(absmax8(yv)));   // all 64 lanes take part
        const uint2 c8 = tiny_scale(sc) ? encode8<true>(yv, sc) : encode8<false>(yv, sc);
        if (ok)
            *reinterpret_cast<uint2 *>(q + row * cols + c) = c8;
        const int64_t g = 4 * p + sub;
        if (li == 0 && p < npass && g < ngc)
            s[row * ngc + g] = sc.s;
    };
    if (NP > 0) {
#pragma unroll
        for (int j = 0; j < NP; ++j)
            if (w + (int64_t)j * SW < npass)   // uniform across the wave
                body(w + (int64_t)j * SW, keep[j]);
    } else {
        for (int64_t p = w; p < npass; p += SW)
            body(p, load(p));
    }
}

// ---------------------------------------------------------------- INT8 W8A8 rows

// 8 int8 codes of one 16-byte bf16 load: clamp(RNE(RN32(x / s)), +-127)
template <bool LIFT>
__device__ __forceinline__ uint2 encode8_i8(const uint4 &v, const Scale &sc)
{
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float n = __builtin_rintf(quot_t<LIFT>(bf16_elem(v, i), sc));   // ties to even
        n = fminf(fmaxf(n, -127.0f), 127.0f);
        w[i >> 2] |= ((uint32_t)(int32_t)n & 0xFFu) << (8 * (i & 3));
    }
    return make_uint2(w[0], w[1]);
}

// One symmetric scale per row (a token of an activation, an output channel of a weight):
// s = RN32(amax / 127).  One wave per row; pass p covers columns 512 p .. 512 p + 511, 16
// bytes per lane.  NP > 0: the row stays in registers (NP passes at most); NP == 0: it is
// read twice.
template <int NP>
__global__ __launch_bounds__(256) void k_quant_int8_rows(const uint16_t *__restrict__ x,
                                                         int64_t rows, int64_t cols, int64_t ldx,
                                                         uint8_t *__restrict__ q,
                                                         float *__restrict__ s)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;   // the whole wave; no barrier follows
    const int64_t npass = (cols + 511) / 512;
    const uint16_t *xr = x + row * ldx;
    auto load = [&](int64_t p) -> uint4 {
        const int64_t c = 512 * p + 8 * lane;   // cols % 8 == 0: an octet is all in or out
        return c < cols ? *reinterpret_cast<const uint4 *>(xr + c) : make_uint4(0, 0, 0, 0);
    };
    uint32_t m = 0;
    uint4 keep[NP > 0 ? NP : 1];
    if (NP > 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            keep[p] = p < npass ? load(p) : make_uint4(0, 0, 0, 0);
            m = umax(m, absmax8(keep[p]));
        }
    } else {
        for (int64_t p = 0; p < npass; ++p)
            m = umax(m, absmax8(load(p)));
    }
    m = row16_max(m);
    m = umax(m, (uint32_t)__shfl_xor((int)m, 16));
    m = umax(m, (uint32_t)__shfl_xor((int)m, 32));
    const Scale sc = scale_of(__fdiv_rn(__uint_as_float(m << 16), 127.0f));
    if (lane == 0)
        s[row] = sc.s;
    const bool lift = tiny_scale(sc);   // uniform across the wave
    auto body = [&](int64_t p, const uint4 &v) {
        const int64_t c = 512 * p + 8 * lane;
        if (c < cols)
            *reinterpret_cast<uint2 *>(q + row * cols + c) =
                lift ? encode8_i8<true>(v, sc) : encode8_i8<false>(v, sc);
    };
    if (NP > 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
            if (p < npass)
                body(p, keep[p]);
    } else {
        for (int64_t p = 0; p < npass; ++p)
            body(p, load(p));
    }
}

// One wave covers 64 consecutive 8-column chunks of a row (1 KB of bf16); the grid's y
// dimension and the 4 waves of a workgroup walk the rows, so each lane forms the reciprocals
// of its 8 columns once and reuses them for every row it folds.
__global__ __launch_bounds__(256) void k_uaq_fold(const uint16_t *w, int64_t n, int64_t k,
                                                  int64_t ldw, const float *__restrict__ s,
                                                  uint16_t *out, int64_t ldo, float *gain)
{
    const int64_t kc = ((int64_t)blockIdx.x * 64 + (threadIdx.x & 63)) * 8;
    if (kc >= k)
        return;
    Fold8 f;
    fold8_setup(s, kc, f);
    auto fold_chunk = [&](const uint4 &v) { return fold8(v, f); };
    const int64_t step = (int64_t)gridDim.y * 4;
    int64_t row = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
    for (; row + 3 * step < n; row += 4 * step) {       // four rows in flight per lane
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = *reinterpret_cast<const uint4 *>(w + (row + u * step) * ldw + kc);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<uint4 *>(out + (row + u * step) * ldo + kc) = fold_chunk(v[u]);
    }
    for (; row < n; row += step) {
        const uint4 v0 = *reinterpret_cast<const uint4 *>(w + row * ldw + kc);
        *reinterpret_cast<uint4 *>(out + row * ldo + kc) = fold_chunk(v0);
    }
    if (gain && blockIdx.y == 0 && threadIdx.x < 64) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            gain[kc + j] = gain[kc + j] * f.s[j];
    }
}

}  // namespace

// Workgroups of a persistent grid for kernel `fn`: the CU count times the workgroups that fit
// on a CU at once (capped), so the whole grid is resident and each workgroup loops.
static int64_t persistent_grid(const void *fn)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    if (per_cu > kQuantWgPerCu)
        per_cu = kQuantWgPerCu;
    return (int64_t)cus * per_cu;
}

template <int MODE>
static hipError_t launch_mode(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t *q, float *s, uint8_t *qT, float *sT, int64_t ntiles,
                              hipStream_t stream)
{
    const int64_t limit = persistent_grid(reinterpret_cast<const void *>(&k_quant_tile<MODE>));
    const dim3 grid((unsigned)(ntiles < limit ? ntiles : limit));
    k_quant_tile<MODE><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s, qT, sT);
    return hipGetLastError();
}

hipError_t launch_quant_tile(int mode, const uint16_t *x, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t *q, float *s, uint8_t *qT, float *sT,
                             hipStream_t stream)
{
    const int64_t ngr = (rows + kTile - 1) / kTile, ngc = (cols + kTile - 1) / kTile;
    if (ngr == 0 || ngc == 0)
        return hipSuccess;
    const int64_t nt = ngr * ngc;
    switch (mode) {
    case QMODE_ROW:
        if (rows <= kSmallRows) {
            const int64_t waves = rows * ((ngc + 3) / 4);
            k_quant_rows_small<<<(unsigned)((waves + 3) / 4), 256, 0, stream>>>(x, rows, cols,
                                                                               ld_x, q, s);
            return hipGetLastError();
        }
        return launch_mode<QMODE_ROW>(x, rows, cols, ld_x, q, s, qT, sT, nt, stream);
    case QMODE_COL:
        return launch_mode<QMODE_COL>(x, rows, cols, ld_x, q, s, qT, sT, nt, stream);
    case QMODE_ROW | QMODE_COL:
        return launch_mode<QMODE_ROW | QMODE_COL>(x, rows, cols, ld_x, q, s, qT, sT, nt, stream);
    case QMODE_BLK:
        return launch_mode<QMODE_BLK>(x, rows, cols, ld_x, q, s, qT, sT, nt, stream);
    case QMODE_BLK | QMODE_BLKT:
        return launch_mode<QMODE_BLK | QMODE_BLKT>(x, rows, cols, ld_x, q, s, qT, sT, nt, stream);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_fold_quant_w(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                               const float *fs, uint16_t *w_out, int64_t ld_out, float *gain,
                               uint8_t *q, float *s, uint8_t *qT, float *sT, hipStream_t stream)
{
    const int64_t nt = ((n + kTile - 1) / kTile) * ((k + kTile - 1) / kTile);
    if (nt == 0)
        return hipSuccess;
    FoldArgs fa;
    fa.s = fs;
    fa.out = w_out;
    fa.ldo = ld_out;
    fa.gain = gain;
    constexpr int BT = QMODE_BLK | QMODE_BLKT | QMODE_FOLD, B = QMODE_BLK | QMODE_FOLD;
    const void *fn = qT ? reinterpret_cast<const void *>(&k_fold_quant_w<BT>)
                        : reinterpret_cast<const void *>(&k_fold_quant_w<B>);
    const int64_t limit = persistent_grid(fn);
    const dim3 grid((unsigned)(nt < limit ? nt : limit));
    if (qT)
        k_fold_quant_w<BT><<<grid, 256, 0, stream>>>(w, n, k, ld_w, q, s, qT, sT, fa);
    else
        k_fold_quant_w<B><<<grid, 256, 0, stream>>>(w, n, k, ld_w, q, s, qT, sT, fa);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_quant_dual(const uint16_t *h, int64_t rows, int64_t cols, int64_t ld_h,
                                     const float *gain, float eps, float *inv, uint16_t *y,
                                     uint8_t *q, float *s, uint8_t *qT, float *sT,
                                     hipStream_t stream)
{
    const int64_t nt = ((rows + kTile - 1) / kTile) * ((cols + kTile - 1) / kTile);
    if (nt == 0)
        return hipSuccess;
    k_rms_inv<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(h, rows, cols, ld_h, eps, inv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    NormArgs na;
    na.inv = inv;
    na.gain = gain;
    na.y = y;
    constexpr int RC = QMODE_ROW | QMODE_COL | QMODE_NORM, R = QMODE_ROW | QMODE_NORM,
                  C = QMODE_COL | QMODE_NORM;
    const int mode = (q ? QMODE_ROW : 0) | (qT ? QMODE_COL : 0) | QMODE_NORM;
    const void *fn = mode == RC ? reinterpret_cast<const void *>(&k_norm_quant_tile<RC>)
                     : mode == R ? reinterpret_cast<const void *>(&k_norm_quant_tile<R>)
                                 : reinterpret_cast<const void *>(&k_norm_quant_tile<C>);
    const int64_t limit = persistent_grid(fn);
    const dim3 grid((unsigned)(nt < limit ? nt : limit));
    if (mode == RC)
        k_norm_quant_tile<RC><<<grid, 256, 0, stream>>>(h, rows, cols, ld_h, q, s, qT, sT, na);
    else if (mode == R)
        k_norm_quant_tile<R><<<grid, 256, 0, stream>>>(h, rows, cols, ld_h, q, s, qT, sT, na);
    else
        k_norm_quant_tile<C><<<grid, 256, 0, stream>>>(h, rows, cols, ld_h, q, s, qT, sT, na);
    return hipGetLastError();
}

hipError_t launch_quant_w_batch(const WeightDesc *descs, int count, bool transposed,
                                hipStream_t stream)
{
    constexpr int BT = QMODE_BLK | QMODE_BLKT, B = QMODE_BLK;
    const int64_t limit = persistent_grid(
        transposed ? reinterpret_cast<const void *>(&k_quant_w_batch<BT>)
                   : reinterpret_cast<const void *>(&k_quant_w_batch<B>));
    for (int i0 = 0; i0 < count; i0 += kMaxWeightBatch) {
        WeightTable tab;
        tab.count = count - i0 < kMaxWeightBatch ? count - i0 : kMaxWeightBatch;
        int64_t total = 0;
        for (int i = 0; i < tab.count; ++i) {
            tab.d[i] = descs[i0 + i];
            total += tab.d[i].tiles;
        }
        const dim3 grid((unsigned)(total < limit ? total : limit));
        if (transposed)
            k_quant_w_batch<BT><<<grid, 256, 0, stream>>>(tab);
        else
            k_quant_w_batch<B><<<grid, 256, 0, stream>>>(tab);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_rmsnorm_quant(const uint16_t *h, int64_t rows, int64_t cols, int64_t ld_h,
                                const float *gain, float eps, uint16_t *y, uint8_t *q, float *s,
                                hipStream_t stream)
{
    if (rows == 0 || cols == 0)
        return hipSuccess;
    const int64_t npass = ((cols + kTile - 1) / kTile + 3) / 4;
    if (rows <= kSmallRows && npass >= 2) {
        // few rows: a workgroup of 8 waves per row instead of one wave
        const dim3 g1((unsigned)rows);
        if (npass <= 8)
            k_rmsnorm_quant_split<1, 8><<<g1, 512, 0, stream>>>(h, rows, cols, ld_h, gain, eps, y, q, s);
        else if (npass <= 64)
            k_rmsnorm_quant_split<8, 8><<<g1, 512, 0, stream>>>(h, rows, cols, ld_h, gain, eps, y, q, s);
        else
            k_rmsnorm_quant_split<0, 8><<<g1, 512, 0, stream>>>(h, rows, cols, ld_h, gain, eps, y, q, s);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (cols == 8 * 512)   // whole passes only
        k_rmsnorm_quant<8, true><<<grid, 256, 0, stream>>>(h, rows, cols, ld_h, gain, eps, y, q, s);
    else if (npass <= 8)
        k_rmsnorm_quant<8, false><<<grid, 256, 0, stream>>>(h, rows, cols, ld_h, gain, eps, y, q, s);
    else if (npass <= 16)
        k_rmsnorm_quant<16, false><<<grid, 256, 0, stream>>>(h, rows, cols, ld_h, gain, eps, y, q, s);
    else
        k_rmsnorm_quant<0, false><<<grid, 256, 0, stream>>>(h, rows, cols, ld_h, gain, eps, y, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_int8_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                                  int8_t *q8, float *s, hipStream_t stream)
{
    if (rows == 0 || cols == 0)
        return hipSuccess;
    uint8_t *q = reinterpret_cast<uint8_t *>(q8);
    const int64_t npass = (cols + 511) / 512;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (npass <= 8)
        k_quant_int8_rows<8><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s);
    else if (npass <= 16)
        k_quant_int8_rows<16><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s);
    else
        k_quant_int8_rows<0><<<grid, 256, 0, stream>>>(x, rows, cols, ld_x, q, s);
    return hipGetLastError();
}

hipError_t launch_uaq_fold(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                           const float *s, uint16_t *w_out, int64_t ld_out, float *gain,
                           hipStream_t stream)
{
    // x: 512-column slabs; y: row groups of 4 waves, about 8 rows per wave (capped so the
    // grid stays within the y limit: the row loop covers the rest).
    const int64_t gx = (k + 511) / 512;
    int64_t gy = (n + 31) / 32;
    if (gy > 65535)
        gy = 65535;
    if (gx == 0 || gy == 0)
        return hipSuccess;
    k_uaq_fold<<<dim3((unsigned)gx, (unsigned)gy), 256, 0, stream>>>(w, n, k, ld_w, s, w_out,
                                                                     ld_out, gain);
    return hipGetLastError();
}

}  // namespace qr
