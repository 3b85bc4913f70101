// Internal launch interface between the C ABI layer (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qr {

// Quantizer tile modes (bit flags).
enum : int {
    QMODE_ROW = 1,    // 1x128 row groups, codes in input layout
    QMODE_COL = 2,    // 128x1 column groups, codes and scales stored transposed
    QMODE_BLK = 4,    // 128x128 blocks, codes in input layout
    QMODE_BLKT = 8,   // 128x128 blocks, transposed copy of codes and scales
    QMODE_FOLD = 16,  // the UAQ fold applied to each tile before it is quantized
    QMODE_NORM = 32,  // the RMSNorm applied to each tile before it is quantized
};

// One pass over x [rows, cols] (ld_x) in 128x128 tiles.
//   ROW:  q [rows, cols], s [rows, ceil(cols/128)]
//   COL:  qT [cols, rows], sT [cols, ceil(rows/128)]
//   BLK:  q [rows, cols], s [ceil(rows/128), ceil(cols/128)]
//   BLKT: qT [cols, rows], sT [ceil(cols/128), ceil(rows/128)]
hipError_t launch_quant_tile(int mode, const uint16_t *x, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t *q, float *s, uint8_t *qT, float *sT,
                             hipStream_t stream);

// UAQ fold and 128x128 quantization in one pass: w_out [n, k] (ld_out) = RN_bf16(w / fs[c]),
// gain[c] = RN32(gain[c] * fs[c]) if gain, then q / s (and qT / sT if qT) of w_out as
// launch_quant_tile's BLK (| BLKT) would produce them.  w_out may equal w (ld_out == ld_w).
hipError_t launch_fold_quant_w(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                               const float *fs, uint16_t *w_out, int64_t ld_out, float *gain,
                               uint8_t *q, float *s, uint8_t *qT, float *sT, hipStream_t stream);

// One weight of a batched 128x128 quantization (BLK, plus BLKT when qT is used).
struct WeightDesc {
    const uint16_t *w;      // bf16 [n, k], leading dimension ld
    int64_t n, k, ld;
    uint8_t *q;             // [n, k]
    float *s;               // [ceil(n/128), ceil(k/128)]
    uint8_t *qT;            // [k, n] or unused
    float *sT;              // [ceil(k/128), ceil(n/128)] or unused
    int64_t tiles;          // ceil(n/128) * ceil(k/128), > 0
};
constexpr int kMaxWeightBatch = 32;   // descriptors per launch (they travel as a kernel argument)
struct WeightTable {
    int count;
    WeightDesc d[kMaxWeightBatch];
};

// Quantizes count weights (all with, or all without, the transposed copy) in launches of up
// to kMaxWeightBatch descriptors.
hipError_t launch_quant_w_batch(const WeightDesc *descs, int count, bool transposed,
                                hipStream_t stream);

// y = RN_bf16(h * gain / sqrt(mean(h^2) + eps)) per row of h [rows, cols] (ld_h); y is
// optional (NULL); q [rows, cols] and s [rows, ceil(cols/128)] are y's 1x128 codes and scales.
hipError_t launch_rmsnorm_quant(const uint16_t *h, int64_t rows, int64_t cols, int64_t ld_h,
                                const float *gain, float eps, uint16_t *y, uint8_t *q, float *s,
                                hipStream_t stream);

// The norm with both activation layouts from one read of h: inv [rows] = 1 / sqrt(mean(h^2) +
// eps) (first pass), then y = RN_bf16((h * inv) * gain) quantized as launch_quant_tile's ROW
// (q, s; may be null) and COL (qT, sT; may be null) modes would quantize it; y optional.
hipError_t launch_rmsnorm_quant_dual(const uint16_t *h, int64_t rows, int64_t cols, int64_t ld_h,
                                     const float *gain, float eps, float *inv, uint16_t *y,
                                     uint8_t *q, float *s, uint8_t *qT, float *sT,
                                     hipStream_t stream);

hipError_t launch_uaq_fold(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                           const float *s, uint16_t *w_out, int64_t ld_out, float *gain,
                           hipStream_t stream);

// A GEMM's launch plan.
struct GemmPlan {
    int cfg;        // tile configuration index
    int split;      // number of K splits (1 = none)
    size_t ws_bytes;
};

// INT8 W8A8: C[m, n] = sa[m] * sb[n] * sum_k A[m, k] B[n, k] (int8 codes, K % 128 == 0).
// With plan.split > 1, ws holds the int32 partials [split][M][N] (plan.ws_bytes).
GemmPlan plan_gemm_i8(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_i8(bool out_bf16, const int8_t *A, const float *sa, const int8_t *B,
                          const float *sb, int64_t M, int64_t N, int64_t K, void *C, void *ws,
                          const GemmPlan &plan, hipStream_t stream);

// 4-bit weights: w [n, k] (ld) -> codes [n, k/2], E4M3 block scales [n, k/16], tensor scale;
// partial: kNvfp4Partials words of scratch (the first pass's maxima).
constexpr int kNvfp4Partials = 1024;
hipError_t launch_quant_nvfp4(const uint16_t *w, int64_t n, int64_t k, int64_t ld, uint8_t *codes,
                              uint8_t *bscale, float *tscale, uint32_t *partial,
                              hipStream_t stream);
// Y [M, N] = t * X [M, K] . dequant(W)^T, X bf16 dense, K % 128 == 0.
hipError_t launch_gemm_w4a16(bool out_bf16, const uint16_t *X, const uint8_t *codes,
                             const uint8_t *bscale, const float *tscale, int64_t M, int64_t N,
                             int64_t K, void *Y, hipStream_t stream);

// One symmetric INT8 scale per row: s [rows], q [rows, cols].
hipError_t launch_quant_int8_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                                  int8_t *q, float *s, hipStream_t stream);

// B-operand scale layouts of the block-scaled GEMM C[m, n] = sum_k A[m, k] B[n, k].
enum : int {
    BSCALE_BLOCK = 0,  // sb [ceil(N/128), K/128]: one scale per 128x128 block of B
    BSCALE_ROW = 1,    // sb [N, K/128]: one scale per row of B and 128-group of K
};

GemmPlan plan_gemm(int bscale, int64_t M, int64_t N, int64_t K);

// Size of the file-scope device scratch that the allocation-free FProp uses for its K-split
// partial sums, and its device address on the current device (looked up on the first call
// per device).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);

// A [M, K] codes, sa [M, K/128]; B [N, K] codes, sb per `bscale`; C [M, N] (out_bf16 ? bf16 : f32).
hipError_t launch_gemm(int bscale, bool out_bf16, const uint8_t *A, const float *sa,
                       const uint8_t *B, const float *sb, int64_t M, int64_t N, int64_t K,
                       void *C, void *ws, const GemmPlan &plan, hipStream_t stream);

}  // namespace qr
