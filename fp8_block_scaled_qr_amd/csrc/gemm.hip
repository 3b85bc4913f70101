// Block-scaled FP8 GEMM for gfx950:  C[m, n] = sum_g sa[m, g] * sb(n, g) * P_g[m, n],
// P_g[m, n] = sum_{k in group g} e4m3(A[m, k]) * e4m3(B[n, k]),  groups of 128 along K.
//
// This is the FProp form of the Jet-RL notes (arXiv 2601.14243v1), section on the
// fine-grained GEMM quantization scheme: the activation is quantized 1x128 along K
// (row-major, one scale per row and group) and the weight 128x128 ("column-major" for
// Y = X W^T, i.e. W[N, K] with K contiguous; one scale per block).  DGrad is the same form on
// the transposed weight copy; WGrad is the same form on the two token-grouped transposed
// operands, where the B scale is per row of B (BSCALE_ROW) instead of per block.
//
// Design for CDNA4 (gfx950):
//   * One K step = one scale group of 128: every 16x16 output sub-tile takes exactly one
//     v_mfma_scale_f32_16x16x128_f8f6f4 (E8M0 scales fixed at 2^0, so the hardware block
//     scaling is neutral) into a fresh fp32 partial, which is then promoted into the fp32
//     accumulator with the group's scale product (one FMA per output per group).
//   * The MFMA takes the B rows as its first operand and the A rows as its second, so each
//     lane's four results are four consecutive n of one m: the A scale is one value per
//     lane per sub-tile, and for per-block B scales the whole wave shares one B scale.
//   * A and B tiles (K-contiguous, 128 bytes per row per step) go from memory straight into
//     LDS (buffer loads with the LDS destination, 1 KB = 8 whole rows per instruction) in a
//     ring of stages, with the 16-byte chunk index XOR-swizzled by the row so that the
//     fragment reads are bank-conflict free.  The next steps' loads are issued before the
//     current step's MFMAs.
//   * Work-group ids are remapped so that each XCD (ids are dealt round-robin to the 8 XCDs)
//     takes a contiguous run of tiles, laid out as near-square blocks whose tiles share A and
//     B panels in that XCD's L2.
//   * Decode batches use 64-row tiles with a four-stage ring, and weights too narrow to give
//     every CU a workgroup also split K across workgroups: partial sums go to a caller
//     workspace and a second kernel adds them in a fixed order.
#include "qr_device.h"
#include "qr_internal.h"

#include <algorithm>
#include <mutex>

// Scratch of the allocation-free FProp entry point: the K-split partial sums [split][M][N]
// (fp32) go here instead of a caller workspace.  One copy per GPU, held until the process
// ends.  In host code this name is only a stand-in for the device object: its device address
// comes from hipGetSymbolAddress (noalloc_scratch below) and only that address is used.
static __device__ __align__(256) uint8_t scratch[qr::kNoAllocScratchBytes];

namespace qr {

namespace {
constexpr int kMaxDevices = 64;
}

hipError_t noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // first call on this device, with it current: its own copy of the array
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;

template <int BM_, int BN_, int WM_, int WN_, int NS_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NS = NS_;                         // LDS stages of the load ring
    static_assert(NS >= 2, "at least two stages");
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;       // wave tile
    static constexpr int IM = TM / 16, JN = TN / 16;       // 16x16 sub-tiles per wave
    static constexpr int CA = BM * 8 / THREADS;            // 16-byte A chunks per thread
    static constexpr int CB = BN * 8 / THREADS;            // 16-byte B chunks per thread
    static_assert((BM / 8) % (WM * WN) == 0 && (BN / 8) % (WM * WN) == 0,
                  "whole 8-row x 8-chunk load units per wave");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
    static_assert((BM * 8) % THREADS == 0 && (BN * 8) % THREADS == 0, "chunk split");
    static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns lie in one 128-block");
};

struct GemmArgs {
    const uint8_t *A;
    const float *sa;
    const uint8_t *B;
    const float *sb;
    void *C;            // output, or the fp32 workspace [split][M][N] when split > 1
    int64_t M, N, K;
    int nk;             // K / 128
    int tilesM, tilesN;
    int split, kgps;    // number of K splits, groups per split
    int krot;           // K-start rotation: > 0 multiplier of the workgroup id, < 0 (negated)
                        // multiplier of the XCD index, 0 none
};

// The promotion of a unit's partial sum runs QR_PROMOTE_LAG MFMAs after the MFMA that made it,
// so the VALU never waits on the MFMA result.
#ifndef QR_PROMOTE_LAG
#define QR_PROMOTE_LAG 3
#endif

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Workgroup barrier for the LDS stage ring, without the memory fence of __syncthreads():
// that fence would also wait for the next steps' global loads still in flight.  Ordering is
// explicit: each wave waits for its own LDS accesses (lgkmcnt(0)) so that the stage it wrote
// is complete and no wave refills a stage another wave still reads; the empty asm statements
// keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained (gfx9)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Tile order: workgroup ids are dealt round-robin to the 8 XCDs, so id b is remapped to
// position (b mod 8) * (nb / 8) + b / 8 and each XCD takes a contiguous run of positions.  The
// positions are then laid out in groups of QR_RASTER_GM tile rows, column by column inside a
// group, so that the tiles an XCD runs at the same time form a near-square block: at each K
// step they read fewer distinct A and B panels through that XCD's L2 (4x8 tiles share 12
// panels where a 2x16 strip of one row band needs 18).
#ifndef QR_RASTER_GM
#define QR_RASTER_GM 4
#endif
__device__ __forceinline__ void tile_of(int pos, int tilesM, int tilesN, int &tm, int &tn)
{
    const int per_group = QR_RASTER_GM * tilesN;
    const int grp = pos / per_group;
    const int m_first = grp * QR_RASTER_GM;
    const int rows = min(QR_RASTER_GM, tilesM - m_first);
    const int idx = pos - grp * per_group;
    tm = m_first + idx % rows;
    tn = idx / rows;
}

#ifndef QR_SCALE_CHUNK
#define QR_SCALE_CHUNK 4
#endif

// K-start rotation for weight-streaming launches: a workgroup starts its K walk at a step set
// by its id times this multiplier.  Used where the tiles form one row band and K is not split
// (decode batches): every workgroup then streams its own weight rows, and without the rotation
// all of them read the same 128-byte column of rows 4 KB or more apart at the same time,
// which the memory system serves more slowly than spread offsets (64x14336x4096: 21.6 ->
// 20.3 us, 64x28672x4096: 33.4 -> 29.3, 256x55296x5120: 91.2 -> 88.5; event medians after a
// cache-evicting read).  Tiles over several row bands share A and B panels through L2 at
// the same K step, so all tiles of one XCD keep one order (rotated per workgroup,
// 8192x4096x4096 ran 128 -> 154 us); the XCDs, each with its own L2, start at different steps
// (XCD x at x scale chunks before the end: 1-2 % faster on the 8192x4096x4096 GEMMs).
constexpr int kKRotMul = 5;
constexpr int kKRotXcd = 1;

template <class T, int BSCALE, bool OUT_BF16, bool EB = false>
__global__ __launch_bounds__(T::THREADS) void k_gemm(GemmArgs g)
{
    // Scale slots: BM row scales of A, then the B scales (BN row scales, or the tile's
    // per-block scales; a scale load fills 64 slots, extras duplicate the last one).
    constexpr int NSB = BSCALE == BSCALE_ROW ? T::BN : (T::BN >= kGroup ? T::BN / kGroup : 1);
    constexpr int NW = T::WM * T::WN;
    constexpr int NSA_I = T::BM / 64;                               // A-scale loads per chunk
    constexpr int NSB_I = BSCALE == BSCALE_ROW ? T::BN / 64 : 1;    // B-scale loads per chunk
    constexpr int SB_SLOTS = NSB_I * 64;
    static_assert(NSA_I + NSB_I <= NW, "one scale load per wave and chunk at most");
    constexpr int DA = T::BM / 8 / NW, DB = T::BN / 8 / NW;         // 1 KB tile loads per wave
    static_assert(DA * 8 * NW == T::BM && DB * 8 * NW == T::BN, "whole 1 KB loads per wave");
    // Scales are staged SC groups at a time: a slot's SC consecutive groups are one 16-byte load
    // (one memory request per row instead of one per row and group: the scale rows of
    // consecutive tile rows are K/128 * 4 bytes apart, so a per-group load of a tile's row
    // scales touches a different line per row).  Chunk c covers the steps gb + c SC ..; two
    // chunk buffers alternate.  A deeper stage ring (NS > 2) keeps one scale per step.
    constexpr int SC = T::NS == 2 ? QR_SCALE_CHUNK : 1;
    static_assert(SC == 1 || SC == 4, "scale chunk of 1 or 4 groups");
    constexpr int SBUF = SC == 1 ? T::NS : 2;                       // scale buffers
    // EB (two-stage rings, weight-streaming launches): the B tile of step v + 2 is issued
    // halfway through step v instead of at the start of step v + 1.  A wave reads all of a
    // step's B fragments at its start, so after a barrier that follows them the B half of the
    // stage is free; the B loads then have about a step and a half of lead instead of one, for
    // one more barrier per step.
    constexpr bool EARLY_B = EB && T::NS == 2;
    constexpr int EB_AT = T::IM * T::JN / 2 - 1;   // the MFMA after which the barrier sits
    static_assert(!EARLY_B || EB_AT >= 0, "early B needs MFMAs in the step");

    // Two LDS stages per operand; the global loads write them directly (no register staging).
    // The stages, one block: A stages then B stages.  After the K loop the block holds the
    // bf16 output tile on its way out (the epilogue below).
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::NS * (T::BM + T::BN) * kGroup];
    auto smA = reinterpret_cast<uint8_t (*)[T::BM * kGroup]>(smem);
    auto smB = reinterpret_cast<uint8_t (*)[T::BN * kGroup]>(smem + T::NS * T::BM * kGroup);
    __shared__ __attribute__((aligned(256))) float sS[SBUF][(T::BM + SB_SLOTS) * SC];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index: uniform across the wave, so say so (scalar offsets stay scalar)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int lq = lane >> 4, lr = lane & 15;

    // ---- which tile and K range
    int bid = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0)
        bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    const int tiles = g.tilesM * g.tilesN;
    const int split = bid / tiles;
    const int tile = bid - split * tiles;
    int tm, tn;
    tile_of(tile, g.tilesM, g.tilesN, tm, tn);
    const int64_t m0 = (int64_t)tm * T::BM, n0 = (int64_t)tn * T::BN;
    const int gb = split * g.kgps;
    const int ge = min(g.nk, gb + g.kgps);
    const int64_t M = g.M, N = g.N, K = g.K;
    const int nk = g.nk;

    // ---- LDS layout: row-major, 128 bytes per row, with the 16-byte chunk c of row r stored
    // in slot c ^ f(r), f(r) = (r % 8) ^ ((r / 8) % 2).  A global load instruction fills one
    // contiguous 1 KB block, 8 rows x 128 bytes: lane i writes slot i % 8 of row i / 8, so it
    // reads chunk (i % 8) ^ f(row) -- each row is one whole 128-byte line from memory.  An
    // MFMA operand fragment (lane l: row l % 16, chunks 2 (l / 16) and 2 (l / 16) + 1) is
    // then read with every 8 and every 16 consecutive lanes on distinct 16-byte bank groups
    // (measured as fast as a linear read on gfx950).
    auto swz = [](int row) { return (row & 7) ^ ((row >> 3) & 1); };
    const int frow = lane & 15, fq = lane >> 4;
    const int frag_lo = frow * 128 + (((2 * fq) ^ swz(frow)) << 4);
    const int frag_hi = frow * 128 + (((2 * fq + 1) ^ swz(frow)) << 4);

    // ---- global loads, straight into LDS.  Each operand tile has a buffer descriptor whose
    // range ends at its last valid row, so rows past M or N load zeros.
    const int64_t rowsA = M - m0 < T::BM ? M - m0 : T::BM;
    const int64_t rowsB = N - n0 < T::BN ? N - n0 : T::BN;
    const v4i_sgpr rA = make_rsrc_sgpr(g.A + m0 * K, (uint32_t)(rowsA * K));
    const v4i_sgpr rB = make_rsrc_sgpr(g.B + n0 * K, (uint32_t)(rowsB * K));
    const v4i_sgpr rSA = make_rsrc_sgpr(g.sa + m0 * nk, (uint32_t)(rowsA * nk * 4));
    // per-row B scales: rows n0.. of sb; per-block B scales: block rows n0/128.. of sb
    const int64_t sbRow0 = BSCALE == BSCALE_ROW ? n0 : n0 / kGroup;
    const int64_t sbRows = BSCALE == BSCALE_ROW ? rowsB
                           : ((n0 + rowsB + kGroup - 1) / kGroup) - n0 / kGroup;
    const v4i_sgpr rSB = make_rsrc_sgpr(g.sb + sbRow0 * nk, (uint32_t)(sbRows * nk * 4));
    // tile loads: wave w issues loads t = w + j * NW (rows 8 t .. 8 t + 7)
    const int lrow = lane >> 3, lslot = lane & 7;
    auto tile_voff = [&](int t) -> uint32_t {
        const int row = 8 * t + lrow;
        return (uint32_t)(row * K + ((lslot ^ swz(row)) << 4));
    };
    // scale loads: wave w < NSA_I loads A row scales 64 w .. 64 w + 63, wave NSA_I + s loads
    // B scale slots 64 s .. (rows or blocks, clamped to the last valid index)
    const bool sA_wave = wave < NSA_I, sB_wave = !sA_wave && wave < NSA_I + NSB_I;
    const int sidx = sA_wave ? 64 * wave + lane : min(64 * (wave - NSA_I) + lane, NSB - 1);
    const uint32_t soff = (uint32_t)(sidx * nk * 4);
    const int sdst = sA_wave ? 64 * wave : T::BM + 64 * (wave - NSA_I);

    const uint32_t ldsA = lds_addr_of(&smA[0][0]), ldsB = lds_addr_of(&smB[0][0]);
    const uint32_t ldsS = lds_addr_of(&sS[0][0]);
    const v4i_sgpr rS = sA_wave ? rSA : rSB;
    // The K range is walked from a rotated start: step v of the range [gb, ge) takes group
    // gb + (v + rot) mod len.  Workgroups (or XCDs) that started together then read different
    // K offsets of their rows instead of the same 128-byte column of every row at once.  Ids
    // are dealt round-robin to the 8 XCDs, so blockIdx.x % 8 is the XCD.
    const int len = __builtin_amdgcn_readfirstlane(ge - gb);   // uniform
    int rot = 0;
    if (g.krot != 0 && len > 1) {
        const uint32_t h = g.krot > 0 ? (uint32_t)blockIdx.x * (uint32_t)g.krot
                                      : (blockIdx.x & 7u) * (uint32_t)(-g.krot);
        if (SC == 1) {
            rot = (int)(h % (uint32_t)len);
        } else {
            // the wrap must fall on a scale-chunk boundary: len - rot is a multiple of SC
            const int j = (int)(h % (uint32_t)(len / SC + 1));
            rot = (len - SC * j) % len;
        }
        rot = __builtin_amdgcn_readfirstlane(rot);   // uniform: keep the step walk scalar
    }
    auto grp = [&](int v) {
        const int x = v + rot;
        return gb + (x >= len ? x - len : x);
    };
    // v: the step whose tiles go to stage st (steps past the range re-load the last step's
    // group into a stage that is never read); the step also decides the scale chunk
    auto issue_b = [&](int v, int st) {
        const uint32_t k0 = (uint32_t)grp(min(v, len - 1)) * kGroup;
#pragma unroll
        for (int j = 0; j < DB; ++j) {
            const int t = wave + j * NW;
            dma16(rB, ldsB + (uint32_t)(st * T::BN * kGroup + t * 1024), tile_voff(t) + k0);
        }
    };
    // the A tile and the scales of step v (with EARLY_B the B tile goes separately)
    auto issue_a = [&](int v, int st) {
        const int kg = grp(min(v, len - 1));
        const uint32_t k0 = (uint32_t)kg * kGroup;
#pragma unroll
        for (int j = 0; j < DA; ++j) {
            const int t = wave + j * NW;
            dma16(rA, ldsA + (uint32_t)(st * T::BM * kGroup + t * 1024), tile_voff(t) + k0);
        }
        if (!EARLY_B)
            issue_b(v, st);
        if (SC == 1) {
            if (sA_wave || sB_wave)
                dma4(rS, ldsS + (uint32_t)((st * (T::BM + SB_SLOTS) + sdst) * 4),
                     soff + (uint32_t)kg * 4);
        } else if ((sA_wave || sB_wave) && (v & (SC - 1)) == 0 && v < len) {
            // the chunk of groups kg .. kg + SC - 1, consecutive because the rotation wraps on
            // a chunk boundary (groups past the range are loaded but never read; past the
            // buffer they read as zeros)
            const int c = v / SC;
            dma16(rS, ldsS + (uint32_t)(((c & 1) * (T::BM + SB_SLOTS) + sdst) * SC * 4),
                  soff + (uint32_t)kg * 4);
        }
    };

    v4f acc[T::IM][T::JN];
#pragma unroll
    for (int i = 0; i < T::IM; ++i)
#pragma unroll
        for (int j = 0; j < T::JN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Operand fragment of the 16-row sub-tile starting at (uniform) row r0.
    auto frag = [&](const uint8_t *tileBase, int r0) -> v8i {
        const uint8_t *p = tileBase + r0 * 128;
        const uint4 lo = *reinterpret_cast<const uint4 *>(p + frag_lo);
        const uint4 hi = *reinterpret_cast<const uint4 *>(p + frag_hi);
        v8i f;
        f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
        f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
        return f;
    };

    // compute(stage): the MFMAs of one K step from an LDS stage, with the promotions.  The
    // fragments of the first MFMA are read first, then the other B fragments, then the
    // scales (first needed by the first promotion): every wave starts the step at the same
    // barrier, so the first MFMA should wait for as few LDS reads as possible.
    // tS: the scale buffer; q: the step's column in it (slot r of group q at tS[r SC + q])
    auto compute = [&](const uint8_t *tA, const uint8_t *tB, const float *tS, int q, auto &&mid) {
        const float *tSA = tS + q, *tSB = tS + T::BM * SC + q;
        v8i bf[T::JN];
        v8i afb[2];
        bf[0] = frag(tB, wn * T::TN);
        afb[0] = frag(tA, wm * T::TM);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < T::JN; ++j)
            bf[j] = frag(tB, wn * T::TN + j * 16);
        __builtin_amdgcn_sched_barrier(0);
        float sav[T::IM];
#pragma unroll
        for (int i = 0; i < T::IM; ++i)
            sav[i] = tSA[(wm * T::TM + i * 16 + lr) * SC];
        float sbw = 0.0f;
        float sbv[T::JN][4];
        if (BSCALE == BSCALE_ROW) {
#pragma unroll
            for (int j = 0; j < T::JN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sbv[j][r] = tSB[(wn * T::TN + j * 16 + 4 * lq + r) * SC];
        } else {
            // this wave's 128-column block within the tile (the tile starts on a block
            // boundary or lies inside one block)
            sbw = tSB[(T::BN >= kGroup ? (wn * T::TN) / kGroup : 0) * SC];
        }
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        // Software pipeline over single MFMAs (one M sub-tile x one N sub-tile): the partial
        // of unit u is promoted QR_PROMOTE_LAG units later, so the VALU never waits on it.
        constexpr int NP = QR_PROMOTE_LAG + 1;   // partial buffers
        v4f pbuf[NP];
        auto promote = [&](int u) {
            const int i = u / T::JN, j = u % T::JN;
            const float ci = sav[i] * sbw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float c = BSCALE == BSCALE_ROW ? sav[i] * sbv[j][r] : ci;
                acc[i][j][r] = __builtin_fmaf(pbuf[u % NP][r], c, acc[i][j][r]);
            }
        };
        // A fragments double-buffered: sub-tile i+1's fragment is read from LDS while
        // sub-tile i's MFMAs run, so the LDS latency stays hidden.
#pragma unroll
        for (int u = 0; u < T::IM * T::JN; ++u) {
            const int i = u / T::JN, j = u % T::JN;
            if (j == 0 && i + 1 < T::IM)
                afb[(i + 1) & 1] = frag(tA, wm * T::TM + (i + 1) * 16);
            pbuf[u % NP] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], afb[i & 1], zero,
                                                                           0, 0, 0, 127, 0, 127);
            if (u >= QR_PROMOTE_LAG)
                promote(u - QR_PROMOTE_LAG);
            if (EARLY_B && u == EB_AT)
                mid();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = T::IM * T::JN - QR_PROMOTE_LAG; u < T::IM * T::JN; ++u)
            promote(u);
    };

    // ---- main loop: one 128-wide scale group per step, a ring of NS LDS stages.  Step k
    // first issues the loads of step k+NS-1 into the stage step k-1 used (free: every wave
    // finished reading it before the last barrier), then computes from its own stage; before
    // the barrier each wave waits for its own loads of step k+1 (loads retire in order, so it
    // lets the NS-2 later steps' loads stay in flight), so after it the next stage is
    // complete.  Past the end of the K range the loads re-read the last group (clamped) into
    // stages that are never read.  With two stages the B tiles run further ahead (EARLY_B):
    // step k issues step k+2's B tile halfway through, into its own stage's B half, and the
    // wait before the barrier leaves those loads in flight (they are the wave's last DB).
#pragma unroll
    for (int p = 0; p < T::NS - 1; ++p)
        issue_a(p, p);
    if (EARLY_B) {
        issue_b(0, 0);
        issue_b(1, 1);
    }
    // this wave's loads per step: its tile loads, plus one scale load on the scale waves
    auto wait_next = [&]() {
        constexpr int C = DA + DB;
        if (EARLY_B) {
            vm_wait<DB>();   // all but the B tile of two steps ahead
        } else if (T::NS == 2) {
            vm_wait<0>();
        } else if (sA_wave || sB_wave) {
            vm_wait<(T::NS - 2) * (C + 1)>();
        } else {
            vm_wait<(T::NS - 2) * C>();
        }
    };
    wait_next();   // step gb's loads
    stage_barrier();
    int st = 0, st_load = T::NS - 1;
#pragma nounroll
    for (int v = 0; v < len; ++v) {
        issue_a(v + T::NS - 1, st_load);
        // EARLY_B: once every wave holds this step's B fragments (they are read at the start
        // of the step), the B half of this stage takes the B tile of step v + 2
        auto mid = [&]() {
            stage_barrier();
            issue_b(v + 2, st);
        };
        if (SC == 1)
            compute(smA[st], smB[st], sS[st], 0, mid);
        else
            compute(smA[st], smB[st], sS[(v / SC) & 1], v & (SC - 1), mid);
        wait_next();   // this wave's loads of step k+1
        stage_barrier();
        st = st + 1 == T::NS ? 0 : st + 1;
        st_load = st_load + 1 == T::NS ? 0 : st_load + 1;
    }
    // with more than two stages the last NS-2 steps' loads (clamped re-reads into stages that
    // are never read) are still in flight: they land before the workgroup's LDS is released
    if (T::NS > 2 || EARLY_B)
        vm_wait<0>();

    // ---- epilogue: lane holds C[m][n..n+3] for each sub-tile
    // bf16 output of 64-column wave tiles: staged through LDS so that the stores are whole
    // lines.  A lane's four values go to row r of the wave's region (128 bytes per row, the
    // 16-byte chunk c at slot c ^ swz(r): conflict-free 8-byte writes), then each lane reads 16
    // bytes back and a store instruction covers 8 rows x 128 bytes instead of 16 rows x 32.
    // Measured on the 8192x4096x4096 GEMMs: FProp 150.4 -> 143.9 us, DGrad 145.9 -> 139.7,
    // WGrad 159.4 -> 155.3, the 32B gate+up at batch 256 100.1 -> 95.1; non-temporal stores took
    // another 1-2 %.  (The same staging for fp32 partial sums did not help the K-split shapes
    // and slowed the bf16 kernels, so those keep the direct stores below.)
    if constexpr (OUT_BF16 && T::TN == 64) {
        static_assert(T::BM * T::BN * 2 <= T::NS * (T::BM + T::BN) * kGroup, "tile fits the stages");
        if (g.split == 1 && (N & 7) == 0) {
            if (T::NS > 2 || EARLY_B)
                stage_barrier();   // every wave's last loads have landed (its vm_wait above)
            uint8_t *ep = smem + wave * (T::TM * 128);
#pragma unroll
            for (int i = 0; i < T::IM; ++i)
#pragma unroll
                for (int j = 0; j < T::JN; ++j) {
                    const int r = i * 16 + lr, c = 2 * j + (lq >> 1);
                    const v4f a = acc[i][j];
                    uint2 o;
                    o.x = f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16);
                    o.y = f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16);
                    *reinterpret_cast<uint2 *>(ep + r * 128 + ((c ^ swz(r)) << 4) + (lq & 1) * 8) = o;
                }
            const int c = lane & 7;
            const int64_t n = n0 + wn * T::TN + c * 8;
#pragma unroll
            for (int it = 0; it < T::TM / 8; ++it) {
                const int r = it * 8 + (lane >> 3);
                const uint4 v = *reinterpret_cast<const uint4 *>(ep + r * 128 + ((c ^ swz(r)) << 4));
                const int64_t m = m0 + wm * T::TM + r;
                if (m < M && n < N)   // non-temporal: the output is not read again here
                    __builtin_nontemporal_store(
                        u32x4_t{v.x, v.y, v.z, v.w},
                        reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(g.C) + m * N + n));
            }
            return;
        }
    }
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < T::IM; ++i) {
        const int64_t m = m0 + wm * T::TM + i * 16 + lr;
        if (m >= M)
            continue;
#pragma unroll
        for (int j = 0; j < T::JN; ++j) {
            const int64_t n = n0 + wn * T::TN + j * 16 + 4 * lq;
            const v4f a = acc[i][j];
            if (g.split > 1 || !OUT_BF16) {
                float *c = reinterpret_cast<float *>(g.C) + (int64_t)split * M * N + m * N + n;
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<float4 *>(c) = make_float4(a[0], a[1], a[2], a[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            c[r] = a[r];
                }
            } else {
                uint16_t *c = reinterpret_cast<uint16_t *>(g.C) + m * N + n;
                if (vec_ok && n + 3 < N) {
                    uint2 o;
                    o.x = f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16);
                    o.y = f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16);
                    *reinterpret_cast<uint2 *>(c) = o;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            c[r] = (uint16_t)f32_to_bf16(a[r]);
                }
            }
        }
    }
}

// Sum the split-K partials in split order (deterministic) and convert.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ ws, int64_t MN,
                                                       int split, void *out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if ((MN & 3) == 0) {
        const int64_t n4 = MN >> 2;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
            float4 s = reinterpret_cast<const float4 *>(ws)[i];
            for (int p = 1; p < split; ++p) {
                const float4 v = reinterpret_cast<const float4 *>(ws + p * MN)[i];
                s.x += v.x;
                s.y += v.y;
                s.z += v.z;
                s.w += v.w;
            }
            if (OUT_BF16) {
                uint2 o;
                o.x = f32_to_bf16(s.x) | (f32_to_bf16(s.y) << 16);
                o.y = f32_to_bf16(s.z) | (f32_to_bf16(s.w) << 16);
                reinterpret_cast<uint2 *>(out)[i] = o;
            } else {
                reinterpret_cast<float4 *>(out)[i] = s;
            }
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += stride) {
            float s = ws[i];
            for (int p = 1; p < split; ++p)
                s += ws[p * MN + i];
            if (OUT_BF16)
                reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)f32_to_bf16(s);
            else
                reinterpret_cast<float *>(out)[i] = s;
        }
    }
}

// ---------------------------------------------------------------- INT8 W8A8 GEMM

struct GemmI8Args {
    const int8_t *A;     // [M, K]
    const float *sa;     // [M]
    const int8_t *B;     // [N, K]
    const float *sb;     // [N]
    void *C;             // [M, N], fp32 or bf16; with split > 1 the int32 partials [split][M][N]
    int64_t M, N, K;
    int nk;              // K / 128
    int tilesM, tilesN;
    int split, kgps;     // K splits across workgroups, groups per split
    int krot;            // K-start rotation multiplier per workgroup id (0: none)
};

typedef int v4i __attribute__((ext_vector_type(4)));

// C[m, n] = sa[m] * sb[n] * sum_k A[m, k] B[n, k] with one symmetric scale per row of each
// operand: the integer sum is exact in the int32 MFMA accumulators (|sum| <= 127^2 K), so the
// MFMAs accumulate in place over all of K and both scales are applied once, in the epilogue.
// Staging is the FP8 GEMM's: 128-byte rows of both operands go straight to swizzled LDS, two
// stages.  A 32-byte fragment (lane l: row l % 16, 16-byte chunks 2 (l / 16) and
// 2 (l / 16) + 1 of the 128-byte K step) feeds two 16x16x64 MFMAs, one per chunk; A and B use
// the same lane-to-K assignment, so together the two cover all 128 K of the step.
template <class T, bool OUT_BF16, bool EB = false>
__global__ __launch_bounds__(T::THREADS) void k_gemm_i8(GemmI8Args g)
{
    constexpr int NW = T::WM * T::WN;
    constexpr int DA = T::BM / 8 / NW, DB = T::BN / 8 / NW;
    static_assert(DA * 8 * NW == T::BM && DB * 8 * NW == T::BN, "whole 1 KB loads per wave");
    // NS stages of A then NS stages of B, one block (it also stages the bf16 output tile)
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::NS * (T::BM + T::BN) * kGroup];
    auto smA = reinterpret_cast<uint8_t (*)[T::BM * kGroup]>(smem);
    auto smB = reinterpret_cast<uint8_t (*)[T::BN * kGroup]>(smem + T::NS * T::BM * kGroup);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int lq = lane >> 4, lr = lane & 15;

    int bid = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0)
        bid = (bid & 7) * (nb >> 3) + (bid >> 3);   // a contiguous run of tiles per XCD
    const int tiles = g.tilesM * g.tilesN;
    const int split = bid / tiles;
    int tm, tn;
    tile_of(bid - split * tiles, g.tilesM, g.tilesN, tm, tn);
    const int64_t m0 = (int64_t)tm * T::BM, n0 = (int64_t)tn * T::BN;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int gb = split * g.kgps, ge = min(g.nk, gb + g.kgps);   // this split's K groups

    auto swz = [](int row) { return (row & 7) ^ ((row >> 3) & 1); };
    const int frow = lane & 15, fq = lane >> 4;
    const int frag_lo = frow * 128 + (((2 * fq) ^ swz(frow)) << 4);
    const int frag_hi = frow * 128 + (((2 * fq + 1) ^ swz(frow)) << 4);

    const int64_t rowsA = M - m0 < T::BM ? M - m0 : T::BM;
    const int64_t rowsB = N - n0 < T::BN ? N - n0 : T::BN;
    const v4i_sgpr rA = make_rsrc_sgpr(g.A + m0 * K, (uint32_t)(rowsA * K));
    const v4i_sgpr rB = make_rsrc_sgpr(g.B + n0 * K, (uint32_t)(rowsB * K));
    const int lrow = lane >> 3, lslot = lane & 7;
    auto tile_voff = [&](int t) -> uint32_t {
        const int row = 8 * t + lrow;
        return (uint32_t)(row * K + ((lslot ^ swz(row)) << 4));
    };
    const uint32_t ldsA = lds_addr_of(&smA[0][0]), ldsB = lds_addr_of(&smB[0][0]);
    // EB: the B tile of step v + 2 goes out halfway through step v, as in the FP8 GEMM
    constexpr bool EARLY_B = EB && T::NS == 2;
    auto issue_b = [&](int kg, int st) {
        const uint32_t k0 = (uint32_t)kg * kGroup;
#pragma unroll
        for (int j = 0; j < DB; ++j) {
            const int t = wave + j * NW;
            dma16(rB, ldsB + (uint32_t)(st * T::BN * kGroup + t * 1024), tile_voff(t) + k0);
        }
    };
    auto issue_step = [&](int kg, int st) {
        const uint32_t k0 = (uint32_t)kg * kGroup;
#pragma unroll
        for (int j = 0; j < DA; ++j) {
            const int t = wave + j * NW;
            dma16(rA, ldsA + (uint32_t)(st * T::BM * kGroup + t * 1024), tile_voff(t) + k0);
        }
        if (!EARLY_B)
            issue_b(kg, st);
    };

    v4i acc[T::IM][T::JN];
#pragma unroll
    for (int i = 0; i < T::IM; ++i)
#pragma unroll
        for (int j = 0; j < T::JN; ++j)
            acc[i][j] = v4i{0, 0, 0, 0};

    struct Frag {
        v4i lo, hi;
    };
    auto frag = [&](const uint8_t *tileBase, int r0) -> Frag {
        const uint8_t *p = tileBase + r0 * 128;
        Frag f;
        f.lo = *reinterpret_cast<const v4i *>(p + frag_lo);
        f.hi = *reinterpret_cast<const v4i *>(p + frag_hi);
        return f;
    };
    auto compute = [&](const uint8_t *tA, const uint8_t *tB, auto &&mid) {
        Frag bf[T::JN];
#pragma unroll
        for (int j = 0; j < T::JN; ++j)
            bf[j] = frag(tB, wn * T::TN + j * 16);
        Frag afb[2];
        afb[0] = frag(tA, wm * T::TM);
        // per sub-tile row i: the JN low-half MFMAs, then the JN high-half ones, so the two
        // MFMAs into one accumulator sit JN instructions apart instead of back to back
#pragma unroll
        for (int i = 0; i < T::IM; ++i) {
            if (i + 1 < T::IM)
                afb[(i + 1) & 1] = frag(tA, wm * T::TM + (i + 1) * 16);
#pragma unroll
            for (int j = 0; j < T::JN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf[j].lo, afb[i & 1].lo,
                                                                   acc[i][j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < T::JN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf[j].hi, afb[i & 1].hi,
                                                                   acc[i][j], 0, 0, 0);
            if (EARLY_B && i == T::IM / 2 - 1)
                mid();
        }
    };

    // main loop: as the FP8 GEMM's (step k issues step k+NS-1's loads into the stage step k-1
    // used, computes, waits for its own loads of step k+1, then the barrier publishes the
    // stage; past the end of the range the loads re-read the last group into stages never read)
    // The K walk starts at a rotated step as in the FP8 GEMM (the integer sums are exact, so
    // the order does not change the result): step v takes group gb + (v + rot) mod len.
    const int len = __builtin_amdgcn_readfirstlane(ge - gb);   // uniform
    const uint32_t h = g.krot > 0 ? (uint32_t)blockIdx.x * (uint32_t)g.krot
                                  : (blockIdx.x & 7u) * (uint32_t)(-g.krot);
    const int rot = g.krot != 0 && len > 1
                        ? __builtin_amdgcn_readfirstlane((int)(h % (uint32_t)len)) : 0;
    auto grp = [&](int v) {
        const int x = min(v, len - 1) + rot;
        return gb + (x >= len ? x - len : x);
    };
    auto wait_next = [&]() {
        if (EARLY_B)
            vm_wait<DB>();   // all but the B tile of two steps ahead
        else if (T::NS == 2)
            vm_wait<0>();
        else
            vm_wait<(T::NS - 2) * (DA + DB)>();
    };
    if (len > 0) {
#pragma unroll
        for (int p = 0; p < T::NS - 1; ++p)
            issue_step(grp(p), p);
        if (EARLY_B) {
            issue_b(grp(0), 0);
            issue_b(grp(1), 1);
        }
    }
    wait_next();
    stage_barrier();
    int st = 0, st_load = T::NS - 1;
#pragma nounroll
    for (int v = 0; v < len; ++v) {
        issue_step(grp(v + T::NS - 1), st_load);
        auto mid = [&]() {
            stage_barrier();
            issue_b(grp(v + 2), st);
        };
        compute(smA[st], smB[st], mid);
        wait_next();
        stage_barrier();
        st = st + 1 == T::NS ? 0 : st + 1;
        st_load = st_load + 1 == T::NS ? 0 : st_load + 1;
    }
    if (T::NS > 2 || EARLY_B) {
        vm_wait<0>();      // the last steps' re-reads land before the stages are reused
        stage_barrier();
    }

    // epilogue: lane holds C[m][n .. n + 3] of each sub-tile
    // bf16 output of 64-column wave tiles: staged through LDS and stored as whole lines, as
    // in the FP8 GEMM
    if constexpr (OUT_BF16 && T::TN == 64) {
        static_assert(T::BM * T::BN * 2 <= T::NS * (T::BM + T::BN) * kGroup, "tile fits the stages");
        if (g.split == 1 && (N & 7) == 0) {
            uint8_t *ep = smem + wave * (T::TM * 128);
#pragma unroll
            for (int i = 0; i < T::IM; ++i) {
                const int64_t m = m0 + wm * T::TM + i * 16 + lr;
                const float am = m < M ? g.sa[m] : 0.0f;
#pragma unroll
                for (int j = 0; j < T::JN; ++j) {
                    const int64_t n = n0 + wn * T::TN + j * 16 + 4 * lq;
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = n + r < N ? (float)acc[i][j][r] * (am * g.sb[n + r]) : 0.0f;
                    const int rr = i * 16 + lr, c = 2 * j + (lq >> 1);
                    uint2 o;
                    o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
                    o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
                    *reinterpret_cast<uint2 *>(ep + rr * 128 + ((c ^ swz(rr)) << 4) + (lq & 1) * 8) = o;
                }
            }
            const int c = lane & 7;
            const int64_t n = n0 + wn * T::TN + c * 8;
#pragma unroll
            for (int it = 0; it < T::TM / 8; ++it) {
                const int r = it * 8 + (lane >> 3);
                const uint4 v = *reinterpret_cast<const uint4 *>(ep + r * 128 + ((c ^ swz(r)) << 4));
                const int64_t m = m0 + wm * T::TM + r;
                if (m < M && n < N)
                    __builtin_nontemporal_store(
                        u32x4_t{v.x, v.y, v.z, v.w},
                        reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(g.C) + m * N + n));
            }
            return;
        }
    }
    const bool vec_ok = (N & 3) == 0;
    if (g.split > 1) {
        // this split's exact int32 partial sums; the scales are applied once, after the sum
#pragma unroll
        for (int i = 0; i < T::IM; ++i) {
            const int64_t m = m0 + wm * T::TM + i * 16 + lr;
            if (m >= M)
                continue;
#pragma unroll
            for (int j = 0; j < T::JN; ++j) {
                const int64_t n = n0 + wn * T::TN + j * 16 + 4 * lq;
                int32_t *c = reinterpret_cast<int32_t *>(g.C) + (int64_t)split * M * N + m * N + n;
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<v4i *>(c) = acc[i][j];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            c[r] = acc[i][j][r];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < T::IM; ++i) {
        const int64_t m = m0 + wm * T::TM + i * 16 + lr;
        if (m >= M)
            continue;
        const float am = g.sa[m];
#pragma unroll
        for (int j = 0; j < T::JN; ++j) {
            const int64_t n = n0 + wn * T::TN + j * 16 + 4 * lq;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = n + r < N ? (float)acc[i][j][r] * (am * g.sb[n + r]) : 0.0f;
            if (!OUT_BF16) {
                float *c = reinterpret_cast<float *>(g.C) + m * N + n;
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<float4 *>(c) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            c[r] = v[r];
                }
            } else {
                uint16_t *c = reinterpret_cast<uint16_t *>(g.C) + m * N + n;
                if (vec_ok && n + 3 < N) {
                    uint2 o;
                    o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
                    o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
                    *reinterpret_cast<uint2 *>(c) = o;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            c[r] = (uint16_t)f32_to_bf16(v[r]);
                }
            }
        }
    }
}

// Sum the INT8 GEMM's int32 K-split partials in split order (exact) and apply the row scales as
// the unsplit epilogue does, so the output is the same as without the split.  Each thread takes
// four adjacent outputs of one row when N % 4 == 0, else one.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_splitk_reduce_i8(const int32_t *__restrict__ ws,
                                                          int64_t M, int64_t N, int split,
                                                          const float *__restrict__ sa,
                                                          const float *__restrict__ sb, void *out)
{
    const int64_t MN = M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if ((N & 3) == 0) {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN / 4; i += stride) {
            v4i t = reinterpret_cast<const v4i *>(ws)[i];
            for (int p = 1; p < split; ++p)
                t += reinterpret_cast<const v4i *>(ws + p * MN)[i];
            const int64_t m = (4 * i) / N, n = 4 * i - m * N;
            const float am = sa[m];
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = (float)t[r] * (am * sb[n + r]);
            if (OUT_BF16) {
                uint2 o;
                o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
                o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
                reinterpret_cast<uint2 *>(out)[i] = o;
            } else {
                reinterpret_cast<float4 *>(out)[i] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
        return;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += stride) {
        int32_t t = ws[i];
        for (int p = 1; p < split; ++p)
            t += ws[p * MN + i];
        const int64_t m = i / N, n = i - m * N;
        const float v = (float)t * (sa[m] * sb[n]);
        if (OUT_BF16)
            reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)f32_to_bf16(v);
        else
            reinterpret_cast<float *>(out)[i] = v;
    }
}

// Tile configurations, indexed by GemmPlan::cfg.
using CfgBig4 = TileCfg<256, 256, 2, 4>;   // prefill / training: 8 waves, 128x64 per wave
using CfgM64 = TileCfg<64, 128, 1, 4>;     // M <= 64 with per-row B scales
using CfgW128 = TileCfg<256, 128, 4, 2>;   // decode, M <= 256 with large splits: 64x64 per wave
// Decode batches of at most 64 rows with per-block B scales: 64-row tiles whose four-stage ring
// keeps three groups of loads in flight (the weight is streamed once; deeper rings measured
// slower), 64 weight rows per workgroup, or 128 when 64-wide tiles would need more than one
// wave of workgroups (the 8B gate+up projection, 28672 rows: 37.7 -> 33.1 us).
using CfgDec64 = TileCfg<64, 64, 1, 4, 4>;     // 4 waves of 64x16
using CfgDec128 = TileCfg<64, 128, 1, 8, 4>;   // 8 waves of 64x16

enum { CFG_M64 = 1, CFG_BIG4 = 4, CFG_DEC64 = 5, CFG_W128 = 6, CFG_DEC128 = 7 };
// INT8 GEMM for decode-sized M: the FP8 decode tiles, 64x64 with 4 waves (64x16 each) and a
// four-stage ring.  Against the earlier 64x32 two-wave, two-stage tiles (event medians after a
// cache-evicting read): 64x14336x4096 29.7 -> 20.6 us, 64x4096x14336 46.9 -> 20.0, 16x14336x4096
// 28.3 -> 18.2, 64x28672x4096 37.6 -> 34.6; 64x32 tiles with four stages were in between.
using CfgI8Small = TileCfg<64, 64, 1, 4, 4>;

void tile_dims(int cfg, int &bm, int &bn)
{
    switch (cfg) {
    case CFG_BIG4: bm = CfgBig4::BM; bn = CfgBig4::BN; break;
    case CFG_W128: bm = CfgW128::BM; bn = CfgW128::BN; break;
    case CFG_DEC64: bm = CfgDec64::BM; bn = CfgDec64::BN; break;
    case CFG_DEC128: bm = CfgDec128::BM; bn = CfgDec128::BN; break;
    default: bm = CfgM64::BM; bn = CfgM64::BN; break;
    }
}

template <class T, int BSCALE, bool OUT_BF16, bool EB = false>
hipError_t launch_cfg(const GemmArgs &a, int blocks, hipStream_t stream)
{
    k_gemm<T, BSCALE, OUT_BF16, EB><<<blocks, T::THREADS, 0, stream>>>(a);
    return hipGetLastError();
}

// The early B loads (EB) serve launches whose tiles form one row band (decode batches of up to
// 256 rows streaming a weight: the 32B layer's four linears at batch 256 went 220.9 -> 213.2 us
// in whole-bench A/B runs, gate+up 91.1 -> 85.2 and QKV 34.0 -> 32.0 in isolation).  The
// training GEMMs' tiles share panels through L2 and have their loads in flight longer already;
// there the extra barrier cost about 1 % in the same A/B runs, so they keep one barrier.
template <class T>
hipError_t launch_t(int bscale, bool out_bf16, const GemmArgs &a, int blocks, hipStream_t s)
{
    if (bscale == BSCALE_ROW)
        return out_bf16 ? launch_cfg<T, BSCALE_ROW, true>(a, blocks, s)
                        : launch_cfg<T, BSCALE_ROW, false>(a, blocks, s);
    if constexpr (T::NS == 2) {
        if (a.tilesM == 1)
            return out_bf16 ? launch_cfg<T, BSCALE_BLOCK, true, true>(a, blocks, s)
                            : launch_cfg<T, BSCALE_BLOCK, false, true>(a, blocks, s);
    }
    return out_bf16 ? launch_cfg<T, BSCALE_BLOCK, true>(a, blocks, s)
                    : launch_cfg<T, BSCALE_BLOCK, false>(a, blocks, s);
}

}  // namespace

constexpr int64_t kCUs = 256;   // MI355X compute units: one 256x256 workgroup each

// Fewest K groups per split on the 256-row tiles.
constexpr int64_t kMinSplitGroups = 3;
// Most K steps per workgroup of the 256-row tiles for which a product moves to the decode tiles.
constexpr int64_t kShortKSteps = 6;

GemmPlan plan_gemm(int bscale, int64_t M, int64_t N, int64_t K)
{
    GemmPlan p;
    // M > 64: 256x256 tiles, 8 waves of 128x64 (the per-row B scales of WGrad fit too, now
    // that the operand tiles go straight from memory to LDS without register staging).  At
    // decode batches of 65..256 rows this reads each weight panel once for all rows, where
    // 128x128 or 256x64 tiles re-read the whole activation for every 128 or 64 weight rows
    // (2.1x faster on a 32B layer's four linears at batch 256).
    // Decode batches of 65..256 rows whose 256x256 tiles would need a K split so large that
    // the fp32 partial sums (split * M * N * 4 bytes) outweigh the weight (N * K bytes): 256x128
    // tiles, twice as many, so half the split and half the partials.  On a 32B layer at batch
    // 256: QKV 37.9 -> 33.6 us, O 34.4 -> 28.9 us; the down projection (K = 27648, partials
    // 0.44x its weight) stays on 256x256 tiles (63.6 against 71.5 us on 256x128).
    bool mid = false;
    if (M > 64) {
        p.cfg = CFG_BIG4;
        const int64_t big = ((M + 255) / 256) * ((N + 255) / 256), nk0 = K / kGroup;
        if (M <= 256 && bscale == BSCALE_BLOCK && big > 0 && big <= kCUs / 2 && nk0 > 1) {
            const int64_t sp = std::min<int64_t>(kCUs / big, nk0);
            if (sp * M * 4 > K) {
                p.cfg = CFG_W128;
                mid = true;
            }
        }
    } else if (M <= 64 && bscale == BSCALE_BLOCK)
        p.cfg = (N + 63) / 64 > kCUs ? CFG_DEC128 : CFG_DEC64;   // decode: stream B once
    else
        p.cfg = CFG_M64;
    int bm, bn;
    tile_dims(p.cfg, bm, bn);
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t nk = K / kGroup;
    int64_t split = 1;
    // Decode batches on narrow weights: fewer than half of the CUs would get a workgroup, so
    // K is split across workgroups as well (at least 8 groups each, so the load ring stays
    // full; the fp32 partials are small at M <= 64).  A 64x4096x4096 product gets 4 splits.
    const bool dec = p.cfg == CFG_DEC64 || p.cfg == CFG_DEC128;
    if (dec && tiles > 0 && tiles <= kCUs / 2 && nk >= 16) {
        split = kCUs / tiles;
        if (split > nk / 8)
            split = nk / 8;
        const int64_t kgps = (nk + split - 1) / split;
        split = (nk + kgps - 1) / kgps;
    }
    if (p.cfg != CFG_BIG4 && !dec && !mid && tiles > 0 && tiles < 512 &&
        nk > 0) {
        split = (512 + tiles - 1) / tiles;
        const int64_t max_split = nk / 4 > 1 ? nk / 4 : 1;   // keep >= 4 groups per split
        if (split > max_split)
            split = max_split;
        if (split > 16)
            split = 16;
        if (split < 1)
            split = 1;
        const int64_t kgps = (nk + split - 1) / split;
        split = (nk + kgps - 1) / kgps;
    }
    // 256x256 tiles that would leave more than half of the CUs idle: split K so that the
    // tiles' splits make one wave of at most one workgroup per CU (a decode batch of 256 rows
    // against a 7168-wide weight has 28 tiles, 8 splits of 5 groups each), keeping at least
    // kMinSplitGroups groups per split.  With one or two groups a split's ring fill, partial
    // sums and their sum cost more than the parallelism gains (256x4096x1024: 26.9 us on 8
    // splits, 20.0 on 2; 200x2048x896: 18.5 on 7, 16.1 on 2).
    if ((p.cfg == CFG_BIG4 || mid) && tiles > 0 && tiles <= kCUs / 2 && nk > 1) {
        split = std::min<int64_t>(kCUs / tiles, nk / kMinSplitGroups);
        if (split < 1)
            split = 1;
        const int64_t kgps = (nk + split - 1) / split;
        split = (nk + kgps - 1) / kgps;
    }
    // Short K walks on the 256-row tiles: when their workgroups would walk only a few K steps
    // each and K is split (partial sums for a few steps) or there are few of them, the decode
    // tiles (64 rows, a four-stage ring) are faster: 64x64 tiles up to 256 of them, else
    // 64x128.  Event medians after a cache-evicting read, 256-row plan -> decode tiles:
    // 256x512x512 11.0 -> 7.0 us, 1024x1024x1024 23.5 -> 8.8, 2048x2048x2048 36.4 -> 26.1,
    // 4096x2048x1024 36.6 -> 30.2, 1024x4096x512 (64 tiles, unsplit) 15.6 -> 13.9; WGrad with
    // per-row B scales, dW 1024x1024 over 1024 tokens 25.3 -> 9.0, 4096x1024 over 1024 tokens
    // 31.3 -> 18.8.  Unsplit launches with more workgroups keep the 256-row tiles (200x16000x512,
    // 125 workgroups: 11.4 against 13.8; dW 4096x4096 over 512 tokens: 21.7 against 40.8), as do
    // the 32B layer's decode batches (7 or more steps per workgroup).
    const int64_t wgs = tiles * split;
    if (M > 64 && nk > 0 && (nk + split - 1) / split <= kShortKSteps &&
        (split > 1 || wgs <= kCUs / 4)) {
        const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
        p.cfg = t64 <= kCUs ? CFG_DEC64 : CFG_DEC128;
        tile_dims(p.cfg, bm, bn);
        const int64_t t = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        split = 1;
        if (t <= kCUs / 2 && nk >= 16) {   // the decode split rule above
            split = std::min<int64_t>(kCUs / t, nk / 8);
            const int64_t kgps = (nk + split - 1) / split;
            split = (nk + kgps - 1) / kgps;
        }
    }
    p.split = (int)split;
    p.ws_bytes = split > 1 ? (size_t)split * (size_t)M * (size_t)N * sizeof(float) : 0;
    return p;
}

hipError_t launch_gemm(int bscale, bool out_bf16, const uint8_t *A, const float *sa,
                       const uint8_t *B, const float *sb, int64_t M, int64_t N, int64_t K,
                       void *C, void *ws, const GemmPlan &plan, hipStream_t stream)
{
    int bm, bn;
    tile_dims(plan.cfg, bm, bn);
    GemmArgs a;
    a.A = A;
    a.sa = sa;
    a.B = B;
    a.sb = sb;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nk = (int)(K / kGroup);
    a.tilesM = (int)((M + bm - 1) / bm);
    a.tilesN = (int)((N + bn - 1) / bn);
    a.split = plan.split;
    a.kgps = (a.nk + plan.split - 1) / plan.split;
    a.krot = plan.split > 1 ? 0 : a.tilesM == 1 ? kKRotMul : -kKRotXcd;
    a.C = plan.split > 1 ? ws : C;
    const int blocks = a.tilesM * a.tilesN * plan.split;
    hipError_t e;
    switch (plan.cfg) {
    case CFG_DEC64: e = launch_t<CfgDec64>(bscale, out_bf16, a, blocks, stream); break;
    case CFG_DEC128: e = launch_t<CfgDec128>(bscale, out_bf16, a, blocks, stream); break;
    case CFG_BIG4: e = launch_t<CfgBig4>(bscale, out_bf16, a, blocks, stream); break;
    case CFG_W128: e = launch_t<CfgW128>(bscale, out_bf16, a, blocks, stream); break;
    default: e = launch_t<CfgM64>(bscale, out_bf16, a, blocks, stream); break;
    }
    if (e != hipSuccess || plan.split <= 1)
        return e;
    const int64_t MN = M * N;
    int64_t rb = ((MN & 3) == 0 ? MN / 4 : MN + 255) / 256;
    if (rb > 8192)
        rb = 8192;
    if (rb < 1)
        rb = 1;
    if (out_bf16)
        k_splitk_reduce<true><<<(unsigned)rb, 256, 0, stream>>>((const float *)ws, MN, plan.split, C);
    else
        k_splitk_reduce<false><<<(unsigned)rb, 256, 0, stream>>>((const float *)ws, MN, plan.split, C);
    return hipGetLastError();
}

// INT8 plan: cfg 1 = 256x256 tiles, 2 = 256x128 tiles, 0 = 64x64 tiles.  256x256 tiles when they give at least
// half of the CUs a workgroup (prefill and training sizes, and wide weights at decode batches
// up to 256: 256x55296x5120 ran in 110 us instead of 225 on 64x32 tiles).  Below that, M > 64
// still takes 256x256 tiles (each weight panel is read once for all rows) with K split across
// workgroups so that the tiles' splits make one wave of at most one workgroup per CU, as the
// FP8 plan does; M <= 64 takes 64x64 tiles, and splits K only
// when even those leave half of the CUs idle (at least 8 groups per split).
GemmPlan plan_gemm_i8(int64_t M, int64_t N, int64_t K)
{
    GemmPlan p;
    const int64_t nk = K / kGroup;
    const int64_t big_tiles = ((M + CfgBig4::BM - 1) / CfgBig4::BM) * ((N + CfgBig4::BN - 1) / CfgBig4::BN);
    const int64_t small_tiles = ((M + CfgI8Small::BM - 1) / CfgI8Small::BM) *
                                ((N + CfgI8Small::BN - 1) / CfgI8Small::BN);
    p.cfg = big_tiles >= kCUs / 2 || M > 64 ? 1 : 0;
    // As in the FP8 plan: decode batches of 65..256 rows whose 256x256 tiles would split K so
    // far that the int32 partials outweigh the weight take 256x128 tiles (cfg 2), twice the
    // tiles and half the split (the 32B QKV and O at batch 256).
    if (p.cfg == 1 && M <= 256 && big_tiles > 0 && big_tiles <= kCUs / 2 && nk > 1 &&
        std::min<int64_t>(kCUs / big_tiles, nk) * M * 4 > K)
        p.cfg = 2;
    const int64_t mid_tiles = ((M + CfgW128::BM - 1) / CfgW128::BM) *
                              ((N + CfgW128::BN - 1) / CfgW128::BN);
    int64_t split = 1;
    // (at least kMinSplitGroups groups per split, as in the FP8 plan)
    if (p.cfg == 2 && nk > 1) {
        split = std::max<int64_t>(1, std::min<int64_t>(kCUs / mid_tiles, nk / kMinSplitGroups));
    } else if (p.cfg == 1 && big_tiles > 0 && big_tiles < kCUs / 2 && nk > 1) {
        split = std::max<int64_t>(1, std::min<int64_t>(kCUs / big_tiles, nk / kMinSplitGroups));
    } else if (p.cfg == 0 && small_tiles > 0 && small_tiles <= kCUs / 2 && nk >= 16) {
        split = kCUs / small_tiles;
        if (split > nk / 8)
            split = nk / 8;
    }
    if (split > 1) {
        const int64_t kgps = (nk + split - 1) / split;
        split = (nk + kgps - 1) / kgps;
    }
    // Short K walks on the 256-row tiles take the 64x64 tiles instead, as in the FP8 plan (up
    // to 1024 of them: there is no 64x128 INT8 form).  Old plan -> 64x64 tiles, event medians
    // after a cache-evicting read: 256x512x512 16.2 -> 8.6 us, 1024x1024x1024 23.1 -> 10.1,
    // 2048x2048x2048 36.2 -> 27.6, 1024x4096x512 24.6 -> 17.0; 2048x4096x1536 (2048 small
    // tiles) keeps its plan (36.8 against 42.8).
    const int64_t wgs = (p.cfg == 2 ? mid_tiles : big_tiles) * split;
    if (p.cfg != 0 && nk > 0 && (nk + split - 1) / split <= kShortKSteps &&
        (split > 1 || wgs <= kCUs / 4) && small_tiles <= 4 * kCUs) {
        p.cfg = 0;
        split = 1;
        if (small_tiles <= kCUs / 2 && nk >= 16) {   // the 64x64 split rule above
            split = std::min<int64_t>(kCUs / small_tiles, nk / 8);
            const int64_t kgps = (nk + split - 1) / split;
            split = (nk + kgps - 1) / kgps;
        }
    }
    p.split = (int)split;
    p.ws_bytes = split > 1 ? (size_t)split * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
    return p;
}

hipError_t launch_gemm_i8(bool out_bf16, const int8_t *A, const float *sa, const int8_t *B,
                          const float *sb, int64_t M, int64_t N, int64_t K, void *C, void *ws,
                          const GemmPlan &plan, hipStream_t stream)
{
    GemmI8Args a;
    a.A = A;
    a.sa = sa;
    a.B = B;
    a.sb = sb;
    a.C = plan.split > 1 ? ws : C;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nk = (int)(K / kGroup);
    a.split = plan.split;
    a.kgps = (a.nk + plan.split - 1) / plan.split;
    const bool big = plan.cfg == 1, mid = plan.cfg == 2;
    const int bm = big ? CfgBig4::BM : mid ? CfgW128::BM : CfgI8Small::BM;
    const int bn = big ? CfgBig4::BN : mid ? CfgW128::BN : CfgI8Small::BN;
    a.tilesM = (int)((M + bm - 1) / bm);
    a.tilesN = (int)((N + bn - 1) / bn);
    a.krot = plan.split > 1 ? 0 : a.tilesM == 1 ? kKRotMul : -kKRotXcd;
    const unsigned blocks = (unsigned)(a.tilesM * a.tilesN * plan.split);
    const bool eb = a.tilesM == 1;   // one row band: the early B loads (as the FP8 GEMM)
    if (big && eb) {
        if (out_bf16)
            k_gemm_i8<CfgBig4, true, true><<<blocks, CfgBig4::THREADS, 0, stream>>>(a);
        else
            k_gemm_i8<CfgBig4, false, true><<<blocks, CfgBig4::THREADS, 0, stream>>>(a);
    } else if (big) {
        if (out_bf16)
            k_gemm_i8<CfgBig4, true><<<blocks, CfgBig4::THREADS, 0, stream>>>(a);
        else
            k_gemm_i8<CfgBig4, false><<<blocks, CfgBig4::THREADS, 0, stream>>>(a);
    } else if (mid) {
        if (out_bf16)
            k_gemm_i8<CfgW128, true, true><<<blocks, CfgW128::THREADS, 0, stream>>>(a);
        else
            k_gemm_i8<CfgW128, false, true><<<blocks, CfgW128::THREADS, 0, stream>>>(a);
    } else {
        if (out_bf16)
            k_gemm_i8<CfgI8Small, true><<<blocks, CfgI8Small::THREADS, 0, stream>>>(a);
        else
            k_gemm_i8<CfgI8Small, false><<<blocks, CfgI8Small::THREADS, 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.split <= 1)
        return e;
    const int64_t MN = M * N;
    int64_t rb = (((N & 3) == 0 ? MN / 4 : MN) + 255) / 256;
    if (rb > 8192)
        rb = 8192;
    if (rb < 1)
        rb = 1;
    const int32_t *wsi = static_cast<const int32_t *>(ws);
    if (out_bf16)
        k_splitk_reduce_i8<true><<<(unsigned)rb, 256, 0, stream>>>(wsi, M, N, plan.split, sa, sb, C);
    else
        k_splitk_reduce_i8<false><<<(unsigned)rb, 256, 0, stream>>>(wsi, M, N, plan.split, sa, sb, C);
    return hipGetLastError();
}

}  // namespace qr
