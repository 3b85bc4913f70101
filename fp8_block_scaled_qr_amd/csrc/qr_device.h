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

// A group's scale s = RN32(amax / 448) and what the quotient needs: sq = s * m and
// r = RN32(1 / sq), where m = 2^64 for the tiny scales 0 < s < 2^-100 (whose reciprocal could
// overflow and whose residual could underflow) and m = 1 otherwise.  s == 0 (amax == 0) gives
// r = 0.
struct Scale {
    float s;    // the group's scale (the value stored)
    float sq;   // s * m
    float r;    // RN32(1 / sq), 0 when s == 0
    float m;    // 1 or 2^64
};

constexpr float kTinyScale = 0x1p-100f;
constexpr float kTinyLift = 0x1p64f;

__device__ __forceinline__ Scale scale_of(float s)
{
    Scale sc;
    sc.s = s;
    sc.m = (s > 0.0f && s < kTinyScale) ? kTinyLift : 1.0f;
    sc.sq = s * sc.m;
    sc.r = sc.sq == 0.0f ? 0.0f : __fdiv_rn(1.0f, sc.sq);
    return sc;
}

__device__ __forceinline__ Scale make_scale(uint32_t amax_bits15)
{
    return scale_of(__fdiv_rn(__uint_as_float(amax_bits15 << 16), kE4M3Max));
}

__device__ __forceinline__ bool tiny_scale(const Scale &sc) { return sc.m != 1.0f; }

// x / s as the E4M3 encoder needs it: equal to RN32(x / s) bit for bit wherever |x / s| >
// 2^-10, and with the same sign and magnitude <= 2^-10 elsewhere (all of which encode to the
// signed zero).  Method (P. Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990): with r = RN(1/s) and
// q = RN(x*r), the residual x - q*s is exact in one FMA and RN(q + residual*r) is the
// correctly rounded quotient, except where that residual underflows (x tiny, far inside the
// zero code).  The residual is formed as q*s - x and subtracted so that x = -0 yields -0.
// quot() is valid for groups with m == 1 (including s == 0); quot_lifted() for every group:
// it first multiplies x by m, which is exact, so x*m / (s*m) is the same quotient.  A host
// replay of these exact operations over every pair of bf16 amax and bf16 x confirms both
// properties.
__device__ __forceinline__ float quot(float x, const Scale &sc)
{
    float q = x * sc.r;
    float e = __builtin_fmaf(q, sc.sq, -x);
    return __builtin_fmaf(-e, sc.r, q);
}

__device__ __forceinline__ float quot_lifted(float x, const Scale &sc)
{
    return quot(x * sc.m, sc);
}

// Four quotients -> four E4M3 codes (byte i = value i) by the hardware conversion, which
// rounds to nearest even and turns magnitudes above 464 (the midpoint between 448 and the
// next step) into NaN.  A quotient x / s of a finite group never exceeds 448 by more than
// the scale's rounding error (at most ~0.34 %, reached only when amax / 448 is an fp32
// subnormal), so every quotient lies below 464 and the conversion saturates it to +-448 as
// required without a clamp; the conversion's rounding of [448, 464) to 448 is checked on
// the device by the parity tests.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Codes of the 8 bf16 values packed in v (element i in half i%2 of dword i/2), one scale.
// LIFT selects quot_lifted (needed when the group's scale may be tiny).
template <bool LIFT>
__device__ __forceinline__ float quot_t(float x, const Scale &sc)
{
    return LIFT ? quot_lifted(x, sc) : quot(x, sc);
}

template <bool LIFT>
__device__ __forceinline__ uint2 encode8(const uint4 &v, const Scale &sc)
{
    uint2 o;
    o.x = e4m3x4(quot_t<LIFT>(bf16_lo(v.x), sc), quot_t<LIFT>(bf16_hi(v.x), sc),
                 quot_t<LIFT>(bf16_lo(v.y), sc), quot_t<LIFT>(bf16_hi(v.y), sc));
    o.y = e4m3x4(quot_t<LIFT>(bf16_lo(v.z), sc), quot_t<LIFT>(bf16_hi(v.z), sc),
                 quot_t<LIFT>(bf16_lo(v.w), sc), quot_t<LIFT>(bf16_hi(v.w), sc));
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

// ---- raw buffer access and direct-to-LDS loads (gfx9-class descriptors)

// Buffer descriptor word 3 for raw (untyped, stride 0) buffer access on gfx9-class GPUs.
constexpr int kBufFlags = 0x00020000;

// A raw buffer descriptor in four SGPRs: base address, stride 0, extent in bytes, raw-buffer
// flags; offsets at or past the extent read zeros.
typedef int v4i_sgpr __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i_sgpr make_rsrc_sgpr(const void *base, uint32_t extent)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4i_sgpr r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)extent);
    r[3] = kBufFlags;
    return r;
}

// s_waitcnt vmcnt(N): wait until at most N of this wave's vector-memory loads are outstanding
// (they retire in issue order).  Every register an asm load writes must stay live (be named by
// a later asm statement) until the vm_wait that covers the load: the compiler does not know the
// write is still pending and would otherwise reuse the register.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Direct-to-LDS loads issued through inline asm: the buffer load writes lane i's 16 (or 4)
// bytes to LDS address M0 + 16 i (4 i).  The compiler does not see them as memory
// operations, so it adds no waits for them (it cannot tell that they fill the other LDS
// stage and would otherwise wait for them before every read of the current one); the caller
// waits with vm_wait before the barrier that publishes the stage.
//
// M0 is a reserved register, so the compiler warns that naming it as clobbered may not preserve
// it.  That is sound here because no compiler-generated code in these kernels uses M0 at all:
// every M0 instruction in the gfx950 assembly is one of these helpers' own `s_mov_b32 m0`,
// directly before its load (checked on the generated code by tests/test_asm_m0_cpu.py), so
// the warning is silenced for these two statements only.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const v4i_sgpr &rsrc, uint32_t lds_addr, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const v4i_sgpr &rsrc, uint32_t lds_addr, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ object (uniform).
__device__ __forceinline__ uint32_t lds_addr_of(const void *p)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}

}  // namespace qr
