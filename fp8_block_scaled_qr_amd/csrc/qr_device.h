// Device helpers shared by the gfx950 kernels: bf16 unpacking, the exact per-element
// quotient x / s, and the E4M3 encoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qr {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Larger magnitude of the two bf16 halves of w, as a 15-bit pattern.  For finite values the
// integer order of (bits & 0x7FFF) is the order of magnitudes, so no float compare is needed.
__device__ __forceinline__ uint32_t absmax2(uint32_t w)
{
    uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
    return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Max over each row of 16 lanes; every lane of the row receives the result.  All 64 lanes
// must be active.
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    v = umax(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = umax(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = umax(v, dpp<0x141>(v));  // row_half_mirror
    v = umax(v, dpp<0x140>(v));  // row_mirror
    return v;
}

// Group scale s = RN32(amax / 448) and the reciprocal r = RN32(1 / s) used by quot().
struct Scale {
    float s, r;
    bool slow;  // s == 0 or tiny: use the IEEE division path
};

__device__ __forceinline__ Scale make_scale(uint32_t amax_bits15)
{
    Scale sc;
    float amax = __uint_as_float(amax_bits15 << 16);
    sc.s = __fdiv_rn(amax, kE4M3Max);
    sc.r = __fdiv_rn(1.0f, sc.s);
    sc.slow = !(sc.s >= 0x1p-100f);
    return sc;
}

// x / s as the E4M3 encoder needs it: equal to RN32(x / s) bit for bit wherever |x / s| >
// 2^-10, and with the same sign and magnitude <= 2^-10 elsewhere (all of which encode to the
// signed zero).  Fast path (P. Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990): with r = RN(1/s) and
// q = RN(x*r), the residual x - q*s is exact in one FMA and RN(q + residual*r) is the
// correctly rounded quotient, except where that residual underflows (x tiny, far inside the
// zero code).  The residual is formed as q*s - x and subtracted so that x = -0 yields -0.
// Groups whose scale is zero or below 2^-100 (where 1/s may overflow) take the IEEE
// division.  A host replay of these exact operations over every pair of bf16 amax and bf16
// x confirms both properties.
__device__ __forceinline__ float quot(float x, const Scale &sc)
{
    if (sc.slow)
        return sc.s == 0.0f ? x : __fdiv_rn(x, sc.s);
    float q = x * sc.r;
    float e = __builtin_fmaf(q, sc.s, -x);
    return __builtin_fmaf(-e, sc.r, q);
}

// Four values -> four E4M3 codes (byte i = value i): clamp to +-448 (saturation), then the
// hardware round-to-nearest-even conversion.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
    c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
    d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Codes of the 8 bf16 values packed in v (element i in half i%2 of dword i/2), one scale.
__device__ __forceinline__ uint2 encode8(const uint4 &v, const Scale &sc)
{
    uint2 o;
    o.x = e4m3x4(quot(bf16_lo(v.x), sc), quot(bf16_hi(v.x), sc), quot(bf16_lo(v.y), sc),
                 quot(bf16_hi(v.y), sc));
    o.y = e4m3x4(quot(bf16_lo(v.z), sc), quot(bf16_hi(v.z), sc), quot(bf16_lo(v.w), sc),
                 quot(bf16_hi(v.w), sc));
    return o;
}

__device__ __forceinline__ float bf16_elem(const uint4 &v, int i)
{
    uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
}

// float -> bf16, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace qr
