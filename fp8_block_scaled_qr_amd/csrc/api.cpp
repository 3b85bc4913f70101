// C ABI of the gfx950 FP8 quantize-and-multiply library: argument validation (on the host,
// before any HIP call) and dispatch to the kernels.  See include/qr.h for the contract.
#include "qr.h"

#include "qr_internal.h"

#include <algorithm>
#include <vector>

namespace {

constexpr int32_t kAbiVersion = 4;
static_assert(qr::kNoAllocScratchBytes == QR_NOALLOC_SCRATCH_BYTES, "scratch size in qr.h");

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

struct Range {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty if lo == hi
};

Range span(const void *p, int64_t bytes)
{
    Range r;
    if (p && bytes > 0) {
        r.lo = reinterpret_cast<uintptr_t>(p);
        r.hi = r.lo + (uintptr_t)bytes;
    }
    return r;
}

// Bytes spanned by a row-major [rows, cols] tensor with leading dimension ld.
int64_t strided_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t elem)
{
    if (rows <= 0 || cols <= 0)
        return 0;
    return ((rows - 1) * ld + cols) * elem;
}

bool overlap(const Range &a, const Range &b)
{
    return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Products of the sizes must stay far below 2^62; every tensor handled here is < 2^40 bytes.
constexpr int64_t kMaxDim = int64_t(1) << 31;
// Quantizer inputs: a 128-row tile must span less than 2^31 bytes (32-bit buffer offsets).
constexpr int64_t kMaxLd = int64_t(1) << 22;

qr_status launch_status(hipError_t e) { return e == hipSuccess ? QR_OK : QR_ERR_LAUNCH; }

// Argument checks of one 128x128 weight quantization (all but aliasing).
qr_status check_weight(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w, const uint8_t *q,
                       const float *s, const uint8_t *qT, const float *sT)
{
    if (n < 0 || k < 0 || n >= kMaxDim || k >= kMaxDim)
        return QR_ERR_SHAPE;
    if (!q || !s || (qT == nullptr) != (sT == nullptr))
        return QR_ERR_NULL;
    if (n % 8 != 0 || k % 8 != 0 || ld_w % 8 != 0 || (n > 0 && ld_w < k) || ld_w >= kMaxLd)
        return QR_ERR_SHAPE;
    if (cdiv(n, 128) > 65535)
        return QR_ERR_SHAPE;
    if (n == 0 || k == 0)
        return QR_OK;
    if (!w_bf16)
        return QR_ERR_NULL;
    if (misaligned(w_bf16, 16) || misaligned(q, 16) || misaligned(qT, 16) || misaligned(s, 4) ||
        misaligned(sT, 4))
        return QR_ERR_ALIGN;
    return QR_OK;
}

// scratch: the K-split partials go to the library's own device scratch instead of a caller
// workspace (the allocation-free entry point): ws is then unused and the plan's workspace must
// fit the scratch.
qr_status check_gemm(const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                     int64_t M, int64_t N, int64_t K, void *y, int32_t y_dtype, void *ws,
                     size_t ws_bytes, int bscale, int64_t sb_rows, bool scratch = false)
{
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
        return QR_ERR_SHAPE;
    if (K % 128 != 0)
        return QR_ERR_SHAPE;
    if (y_dtype != QR_OUT_F32 && y_dtype != QR_OUT_BF16)
        return QR_ERR_ARG;
    if (M == 0 || N == 0)
        return QR_OK;
    if (!y)
        return QR_ERR_NULL;
    if (K > 0 && (!a || !sa || !b || !sb))
        return QR_ERR_NULL;
    // buffer descriptors address a tile of up to 256 rows with 32-bit offsets
    if (K * 256 >= (int64_t(1) << 31) || (K / 128) * 4 * 256 >= (int64_t(1) << 31))
        return QR_ERR_SHAPE;
    if (misaligned(a, 16) || misaligned(b, 16) || misaligned(y, 16) || misaligned(sa, 4) ||
        misaligned(sb, 4) || misaligned(ws, 16))
        return QR_ERR_ALIGN;
    const int64_t nk = K / 128;
    const int64_t esz = y_dtype == QR_OUT_BF16 ? 2 : 4;
    const qr::GemmPlan plan = qr::plan_gemm(bscale, M, N, K);
    if (scratch) {
        if (plan.ws_bytes > qr::kNoAllocScratchBytes)
            return QR_ERR_SCRATCH;
        ws = nullptr;
    } else if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes)) {
        return QR_ERR_WORKSPACE;
    }
    const Range ry = span(y, M * N * esz);
    const Range rw = span(ws, ws && plan.ws_bytes > 0 ? (int64_t)plan.ws_bytes : 0);
    const Range ins[4] = {span(a, M * K), span(sa, M * nk * 4), span(b, N * K),
                          span(sb, sb_rows * nk * 4)};
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rw, r))
            return QR_ERR_ALIAS;
    if (overlap(ry, rw))
        return QR_ERR_ALIAS;
    return QR_OK;
}

qr_status run_gemm(int bscale, const uint8_t *a, const float *sa, const uint8_t *b,
                   const float *sb, int64_t M, int64_t N, int64_t K, void *y, int32_t y_dtype,
                   void *ws, size_t ws_bytes, qr_stream stream)
{
    const int64_t sb_rows = bscale == qr::BSCALE_ROW ? N : cdiv(N, 128);
    qr_status st = check_gemm(a, sa, b, sb, M, N, K, y, y_dtype, ws, ws_bytes, bscale, sb_rows);
    if (st != QR_OK || M == 0 || N == 0)
        return st;
    // K == 0 (empty contraction) runs the same kernel: no step executes and zeros are stored
    const qr::GemmPlan plan = qr::plan_gemm(bscale, M, N, K);
    return launch_status(qr::launch_gemm(bscale, y_dtype == QR_OUT_BF16, a, sa, b, sb, M, N, K, y,
                                         ws, plan, (hipStream_t)stream));
}

}  // namespace

extern "C" {

const char *qr_status_string(qr_status status)
{
    switch (status) {
    case QR_OK: return "QR_OK";
    case QR_ERR_NULL: return "QR_ERR_NULL: a required pointer is NULL";
    case QR_ERR_SHAPE: return "QR_ERR_SHAPE: a size is negative or violates the entry point's size rules";
    case QR_ERR_ALIGN: return "QR_ERR_ALIGN: a pointer is not aligned as required";
    case QR_ERR_ALIAS: return "QR_ERR_ALIAS: an output overlaps an input or another output";
    case QR_ERR_WORKSPACE: return "QR_ERR_WORKSPACE: the workspace is smaller than required";
    case QR_ERR_LAUNCH: return "QR_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case QR_ERR_ARG: return "QR_ERR_ARG: an enumerated argument is out of range";
    case QR_ERR_SCRATCH:
        return "QR_ERR_SCRATCH: the product's K-split partial sums exceed the allocation-free "
               "entry point's scratch (QR_NOALLOC_SCRATCH_BYTES); use qr_gemm_fp8_bsfprop with a "
               "workspace";
    default: return "unknown qr_status";
    }
}

int32_t qr_abi_version(void) { return kAbiVersion; }

qr_status qr_quant_act_1x128(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t *q_row, float *s_row, uint8_t *q_colT, float *s_colT,
                             qr_stream stream)
{
    if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim)
        return QR_ERR_SHAPE;
    if ((q_row == nullptr) != (s_row == nullptr) || (q_colT == nullptr) != (s_colT == nullptr))
        return QR_ERR_NULL;
    const bool row = q_row != nullptr, col = q_colT != nullptr;
    if (!row && !col)
        return QR_ERR_NULL;
    if (cols % 8 != 0 || ld_x % 8 != 0 || (rows > 0 && ld_x < cols) || (col && rows % 8 != 0) ||
        ld_x >= kMaxLd)
        return QR_ERR_SHAPE;
    if (cdiv(rows, 128) > 65535)
        return QR_ERR_SHAPE;
    if (rows == 0 || cols == 0)
        return QR_OK;
    if (!x_bf16)
        return QR_ERR_NULL;
    if (misaligned(x_bf16, 16) || misaligned(q_row, 16) || misaligned(q_colT, 16) ||
        misaligned(s_row, 4) || misaligned(s_colT, 4))
        return QR_ERR_ALIGN;
    const Range rx = span(x_bf16, strided_bytes(rows, cols, ld_x, 2));
    const Range outs[4] = {span(q_row, rows * cols), span(s_row, rows * cdiv(cols, 128) * 4),
                           span(q_colT, rows * cols), span(s_colT, cols * cdiv(rows, 128) * 4)};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], rx))
            return QR_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j]))
                return QR_ERR_ALIAS;
    }
    const int mode = (row ? qr::QMODE_ROW : 0) | (col ? qr::QMODE_COL : 0);
    return launch_status(qr::launch_quant_tile(mode, static_cast<const uint16_t *>(x_bf16), rows,
                                               cols, ld_x, q_row, s_row, q_colT, s_colT,
                                               (hipStream_t)stream));
}

qr_status qr_rmsnorm_quant_1x128(const void *h_bf16, int64_t rows, int64_t cols, int64_t ld_h,
                                 const float *gain, float eps, void *y_bf16, uint8_t *q_row,
                                 float *s_row, qr_stream stream)
{
    if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim)
        return QR_ERR_SHAPE;
    if (cols % 8 != 0 || ld_h % 8 != 0 || (rows > 0 && ld_h < cols) || ld_h >= kMaxLd)
        return QR_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return QR_ERR_ARG;
    if (rows == 0 || cols == 0)
        return QR_OK;
    if (!h_bf16 || !gain || !q_row || !s_row)
        return QR_ERR_NULL;
    if (misaligned(h_bf16, 16) || misaligned(y_bf16, 16) || misaligned(q_row, 16) ||
        misaligned(gain, 16) || misaligned(s_row, 4))
        return QR_ERR_ALIGN;
    const Range ins[2] = {span(h_bf16, strided_bytes(rows, cols, ld_h, 2)), span(gain, cols * 4)};
    const Range outs[3] = {span(y_bf16, y_bf16 ? rows * cols * 2 : 0), span(q_row, rows * cols),
                           span(s_row, rows * cdiv(cols, 128) * 4)};
    for (int i = 0; i < 3; ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r))
                return QR_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j]))
                return QR_ERR_ALIAS;
    }
    return launch_status(qr::launch_rmsnorm_quant(
        static_cast<const uint16_t *>(h_bf16), rows, cols, ld_h, gain, eps,
        static_cast<uint16_t *>(y_bf16), q_row, s_row, (hipStream_t)stream));
}

qr_status qr_rmsnorm_quant_dual(const void *h_bf16, int64_t rows, int64_t cols, int64_t ld_h,
                                const float *gain, float eps, float *inv_rms, void *y_bf16,
                                uint8_t *q_row, float *s_row, uint8_t *q_colT, float *s_colT,
                                qr_stream stream)
{
    if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim)
        return QR_ERR_SHAPE;
    if ((q_row == nullptr) != (s_row == nullptr) || (q_colT == nullptr) != (s_colT == nullptr))
        return QR_ERR_NULL;
    const bool row = q_row != nullptr, col = q_colT != nullptr;
    if (!row && !col)
        return QR_ERR_NULL;
    if (cols % 8 != 0 || ld_h % 8 != 0 || (rows > 0 && ld_h < cols) || (col && rows % 8 != 0) ||
        ld_h >= kMaxLd || cdiv(rows, 128) > 65535)
        return QR_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return QR_ERR_ARG;
    if (rows == 0 || cols == 0)
        return QR_OK;
    if (!h_bf16 || !gain || !inv_rms)
        return QR_ERR_NULL;
    if (misaligned(h_bf16, 16) || misaligned(y_bf16, 16) || misaligned(q_row, 16) ||
        misaligned(q_colT, 16) || misaligned(gain, 16) || misaligned(s_row, 4) ||
        misaligned(s_colT, 4) || misaligned(inv_rms, 4))
        return QR_ERR_ALIGN;
    const Range ins[2] = {span(h_bf16, strided_bytes(rows, cols, ld_h, 2)), span(gain, cols * 4)};
    const Range outs[6] = {span(inv_rms, rows * 4), span(y_bf16, y_bf16 ? rows * cols * 2 : 0),
                           span(q_row, rows * cols), span(s_row, rows * cdiv(cols, 128) * 4),
                           span(q_colT, rows * cols), span(s_colT, cols * cdiv(rows, 128) * 4)};
    for (int i = 0; i < 6; ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r))
                return QR_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j]))
                return QR_ERR_ALIAS;
    }
    return launch_status(qr::launch_rmsnorm_quant_dual(
        static_cast<const uint16_t *>(h_bf16), rows, cols, ld_h, gain, eps, inv_rms,
        static_cast<uint16_t *>(y_bf16), q_row, s_row, q_colT, s_colT, (hipStream_t)stream));
}

qr_status qr_quant_int8_rowwise(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                int8_t *q, float *s, qr_stream stream)
{
    if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim)
        return QR_ERR_SHAPE;
    if (cols % 8 != 0 || ld_x % 8 != 0 || (rows > 0 && ld_x < cols) || ld_x >= kMaxLd)
        return QR_ERR_SHAPE;
    if (rows == 0 || cols == 0)
        return QR_OK;
    if (!x_bf16 || !q || !s)
        return QR_ERR_NULL;
    if (misaligned(x_bf16, 16) || misaligned(q, 16) || misaligned(s, 4))
        return QR_ERR_ALIGN;
    const Range rx = span(x_bf16, strided_bytes(rows, cols, ld_x, 2));
    const Range rq = span(q, rows * cols), rs = span(s, rows * 4);
    if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs))
        return QR_ERR_ALIAS;
    return launch_status(qr::launch_quant_int8_rows(static_cast<const uint16_t *>(x_bf16), rows,
                                                    cols, ld_x, q, s, (hipStream_t)stream));
}

qr_status qr_gemm_int8_w8a8(const int8_t *a, const float *sa, const int8_t *b, const float *sb,
                            int64_t M, int64_t N, int64_t K, void *y, qr_out_dtype y_dtype,
                            void *workspace, size_t workspace_bytes, qr_stream stream)
{
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
        return QR_ERR_SHAPE;
    if (K % 128 != 0 || K > 131072)   // |sum| <= 127^2 K must fit an int32
        return QR_ERR_SHAPE;
    if (y_dtype != QR_OUT_F32 && y_dtype != QR_OUT_BF16)
        return QR_ERR_ARG;
    if (M == 0 || N == 0)
        return QR_OK;
    if (!sa || !sb || !y || (K > 0 && (!a || !b)))   // K == 0 reads no codes
        return QR_ERR_NULL;
    if (misaligned(a, 16) || misaligned(b, 16) || misaligned(y, 16) || misaligned(sa, 4) ||
        misaligned(sb, 4))
        return QR_ERR_ALIGN;
    const qr::GemmPlan plan = qr::plan_gemm_i8(M, N, K);
    if (plan.ws_bytes > 0) {
        if (!workspace || workspace_bytes < plan.ws_bytes)
            return QR_ERR_WORKSPACE;
        if (misaligned(workspace, 16))
            return QR_ERR_ALIGN;
    }
    const int64_t esz = y_dtype == QR_OUT_BF16 ? 2 : 4;
    const Range ry = span(y, M * N * esz);
    const Range rw = span(workspace, plan.ws_bytes > 0 ? (int64_t)plan.ws_bytes : 0);
    const Range ins[4] = {span(a, M * K), span(sa, M * 4), span(b, N * K), span(sb, N * 4)};
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rw, r))
            return QR_ERR_ALIAS;
    if (overlap(ry, rw))
        return QR_ERR_ALIAS;
    // K == 0 (empty contraction) runs the same kernel: no step executes and zeros are stored
    return launch_status(qr::launch_gemm_i8(y_dtype == QR_OUT_BF16, a, sa, b, sb, M, N, K, y,
                                            workspace, plan, (hipStream_t)stream));
}

qr_status qr_quant_w_nvfp4(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w, uint8_t *codes,
                           uint8_t *bscale, float *tscale, void *workspace,
                           size_t workspace_bytes, qr_stream stream)
{
    if (n < 0 || k < 0 || n >= kMaxDim || k >= kMaxDim)
        return QR_ERR_SHAPE;
    if (k % 32 != 0 || ld_w % 8 != 0 || (n > 0 && ld_w < k) || ld_w >= kMaxLd)
        return QR_ERR_SHAPE;
    if (n == 0 || k == 0)
        return QR_OK;
    if (!w_bf16 || !codes || !bscale || !tscale || !workspace)
        return QR_ERR_NULL;
    if (workspace_bytes < QR_NVFP4_WORKSPACE_BYTES)
        return QR_ERR_WORKSPACE;
    if (misaligned(w_bf16, 16) || misaligned(codes, 16) || misaligned(tscale, 4) ||
        misaligned(workspace, 4))
        return QR_ERR_ALIGN;
    const Range ins[1] = {span(w_bf16, strided_bytes(n, k, ld_w, 2))};
    const Range outs[4] = {span(codes, n * k / 2), span(bscale, n * (k / 16)), span(tscale, 4),
                           span(workspace, QR_NVFP4_WORKSPACE_BYTES)};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], ins[0]))
            return QR_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j]))
                return QR_ERR_ALIAS;
    }
    return launch_status(qr::launch_quant_nvfp4(static_cast<const uint16_t *>(w_bf16), n, k, ld_w,
                                                codes, bscale, tscale,
                                                static_cast<uint32_t *>(workspace),
                                                (hipStream_t)stream));
}

qr_status qr_gemm_w4a16(const void *x_bf16, const uint8_t *codes, const uint8_t *bscale,
                        const float *tscale, int64_t M, int64_t N, int64_t K, void *y,
                        qr_out_dtype y_dtype, qr_stream stream)
{
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
        return QR_ERR_SHAPE;
    if (K % 128 != 0 || cdiv(M, 16) > 65535 || (M + 64) * K * 2 > (int64_t)UINT32_MAX)
        return QR_ERR_SHAPE;
    if (y_dtype != QR_OUT_F32 && y_dtype != QR_OUT_BF16)
        return QR_ERR_ARG;
    if (M == 0 || N == 0)
        return QR_OK;
    if (!x_bf16 || !codes || !bscale || !tscale || !y)
        return QR_ERR_NULL;
    if (misaligned(x_bf16, 16) || misaligned(codes, 16) || misaligned(bscale, 2) ||
        misaligned(tscale, 4) || misaligned(y, 16))
        return QR_ERR_ALIGN;
    const int64_t esz = y_dtype == QR_OUT_BF16 ? 2 : 4;
    const Range ry = span(y, M * N * esz);
    const Range ins[4] = {span(x_bf16, M * K * 2), span(codes, N * K / 2), span(bscale, N * (K / 16)),
                          span(tscale, 4)};
    for (const Range &r : ins)
        if (overlap(ry, r))
            return QR_ERR_ALIAS;
    return launch_status(qr::launch_gemm_w4a16(y_dtype == QR_OUT_BF16,
                                               static_cast<const uint16_t *>(x_bf16), codes,
                                               bscale, tscale, M, N, K, y, (hipStream_t)stream));
}

qr_status qr_quant_w_128x128(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w, uint8_t *q,
                             float *s, uint8_t *qT, float *sT, qr_stream stream)
{
    const qr_status st = check_weight(w_bf16, n, k, ld_w, q, s, qT, sT);
    if (st != QR_OK || n == 0 || k == 0)
        return st;
    const int64_t nblk = cdiv(n, 128) * cdiv(k, 128);
    const Range rw = span(w_bf16, strided_bytes(n, k, ld_w, 2));
    const Range outs[4] = {span(q, n * k), span(s, nblk * 4), span(qT, n * k), span(sT, nblk * 4)};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], rw))
            return QR_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j]))
                return QR_ERR_ALIAS;
    }
    const int mode = qr::QMODE_BLK | (qT ? qr::QMODE_BLKT : 0);
    return launch_status(qr::launch_quant_tile(mode, static_cast<const uint16_t *>(w_bf16), n, k,
                                               ld_w, q, s, qT, sT, (hipStream_t)stream));
}

qr_status qr_quant_w_128x128_batched(const qr_weight_desc *descs, int32_t count,
                                     qr_stream stream)
{
    if (count < 0 || count > QR_MAX_WEIGHT_BATCH)
        return QR_ERR_SHAPE;
    if (count == 0)
        return QR_OK;
    if (!descs)
        return QR_ERR_NULL;
    // every descriptor as for qr_quant_w_128x128, then no output may overlap any input or
    // any other output (inputs may overlap each other)
    struct Tagged {
        Range r;
        bool out;
    };
    std::vector<Tagged> ranges;
    std::vector<qr::WeightDesc> plain, trans;
    for (int32_t i = 0; i < count; ++i) {
        const qr_weight_desc &d = descs[i];
        const qr_status st = check_weight(d.w_bf16, d.n, d.k, d.ld_w, d.q, d.s, d.qT, d.sT);
        if (st != QR_OK)
            return st;
        if (d.n == 0 || d.k == 0)
            continue;
        const int64_t nblk = cdiv(d.n, 128) * cdiv(d.k, 128);
        ranges.push_back({span(d.w_bf16, strided_bytes(d.n, d.k, d.ld_w, 2)), false});
        ranges.push_back({span(d.q, d.n * d.k), true});
        ranges.push_back({span(d.s, nblk * 4), true});
        ranges.push_back({span(d.qT, d.qT ? d.n * d.k : 0), true});
        ranges.push_back({span(d.sT, d.sT ? nblk * 4 : 0), true});
        const qr::WeightDesc w = {static_cast<const uint16_t *>(d.w_bf16), d.n, d.k, d.ld_w,
                                  d.q, d.s, d.qT, d.sT, nblk};
        (d.qT ? trans : plain).push_back(w);
    }
    ranges.erase(std::remove_if(ranges.begin(), ranges.end(),
                                [](const Tagged &t) { return t.r.lo == t.r.hi; }),
                 ranges.end());
    std::sort(ranges.begin(), ranges.end(),
              [](const Tagged &a, const Tagged &b) { return a.r.lo < b.r.lo; });
    // sweep by start address: a range overlaps an earlier one iff it starts below the largest
    // end seen so far (over all ranges if it is an output, over the outputs if it is an input)
    uintptr_t end_all = 0, end_out = 0;
    for (const Tagged &t : ranges) {
        if (t.r.lo < end_out || (t.out && t.r.lo < end_all))
            return QR_ERR_ALIAS;
        end_all = std::max(end_all, t.r.hi);
        if (t.out)
            end_out = std::max(end_out, t.r.hi);
    }
    hipError_t e = hipSuccess;
    if (!plain.empty())
        e = qr::launch_quant_w_batch(plain.data(), (int)plain.size(), false, (hipStream_t)stream);
    if (e == hipSuccess && !trans.empty())
        e = qr::launch_quant_w_batch(trans.data(), (int)trans.size(), true, (hipStream_t)stream);
    return launch_status(e);
}

qr_status qr_gemm_fp8_bsfprop(const uint8_t *a, const float *sa, const uint8_t *b,
                              const float *sb, int64_t M, int64_t N, int64_t K, void *y,
                              qr_out_dtype y_dtype, void *workspace, size_t workspace_bytes,
                              qr_stream stream)
{
    return run_gemm(qr::BSCALE_BLOCK, a, sa, b, sb, M, N, K, y, (int32_t)y_dtype, workspace,
                    workspace_bytes, stream);
}

qr_status qr_gemm_fp8_bsdgrad(const uint8_t *dy, const float *sdy, const uint8_t *wT,
                              const float *swT, int64_t M, int64_t N, int64_t K, void *dx,
                              qr_out_dtype dx_dtype, void *workspace, size_t workspace_bytes,
                              qr_stream stream)
{
    // dX[M, K] = dY[M, N] . W[N, K]: the FProp form with contraction N and B = W^T [K, N]
    return run_gemm(qr::BSCALE_BLOCK, dy, sdy, wT, swT, M, K, N, dx, (int32_t)dx_dtype,
                    workspace, workspace_bytes, stream);
}

qr_status qr_gemm_fp8_bswgrad(const uint8_t *dyT, const float *sdyT, const uint8_t *xT,
                              const float *sxT, int64_t M, int64_t N, int64_t K, void *dw,
                              qr_out_dtype dw_dtype, void *workspace, size_t workspace_bytes,
                              qr_stream stream)
{
    // dW[N, K] = dY^T[N, M] . X[M, K]: the FProp form with contraction M, A = dY^T, B = X^T,
    // and per-row B scales
    return run_gemm(qr::BSCALE_ROW, dyT, sdyT, xT, sxT, N, K, M, dw, (int32_t)dw_dtype,
                    workspace, workspace_bytes, stream);
}

qr_status qr_gemm_fp8_bsfprop_noalloc(const uint8_t *a, const float *sa, const uint8_t *b,
                                      const float *sb, int64_t M, int64_t N, int64_t K, void *y,
                                      qr_out_dtype y_dtype, qr_stream stream)
{
    const int bscale = qr::BSCALE_BLOCK;
    qr_status st = check_gemm(a, sa, b, sb, M, N, K, y, (int32_t)y_dtype, nullptr, 0, bscale,
                              cdiv(N, 128), /*scratch=*/true);
    if (st != QR_OK || M == 0 || N == 0)
        return st;
    const qr::GemmPlan plan = qr::plan_gemm(bscale, M, N, K);
    void *ws = nullptr;
    if (plan.ws_bytes > 0 && qr::noalloc_scratch(&ws) != hipSuccess)
        return QR_ERR_LAUNCH;
    return launch_status(qr::launch_gemm(bscale, y_dtype == QR_OUT_BF16, a, sa, b, sb, M, N, K, y,
                                         ws, plan, (hipStream_t)stream));
}

size_t qr_gemm_workspace_bytes(int32_t kind, int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || K >= kMaxDim || M >= kMaxDim || N >= kMaxDim)
        return 0;
    switch (kind) {
    case QR_GEMM_FPROP:
        return K % 128 || M == 0 || N == 0 || K == 0 ? 0 : qr::plan_gemm(qr::BSCALE_BLOCK, M, N, K).ws_bytes;
    case QR_GEMM_DGRAD:
        return N % 128 || M == 0 || K == 0 || N == 0 ? 0 : qr::plan_gemm(qr::BSCALE_BLOCK, M, K, N).ws_bytes;
    case QR_GEMM_WGRAD:
        return M % 128 || N == 0 || K == 0 || M == 0 ? 0 : qr::plan_gemm(qr::BSCALE_ROW, N, K, M).ws_bytes;
    case QR_GEMM_INT8:
        return K % 128 || K > 131072 || M == 0 || N == 0 || K == 0 ? 0 : qr::plan_gemm_i8(M, N, K).ws_bytes;
    default:
        return 0;
    }
}

qr_status qr_uaq_fold(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w, const float *s,
                      void *w_out_bf16, float *gain_inout, qr_stream stream)
{
    if (n < 0 || k < 0 || n >= kMaxDim || k >= kMaxDim)
        return QR_ERR_SHAPE;
    if (k % 8 != 0 || ld_w % 8 != 0 || (n > 0 && ld_w < k))
        return QR_ERR_SHAPE;
    if (n == 0 || k == 0)
        return QR_OK;
    if (!w_bf16 || !s || !w_out_bf16)
        return QR_ERR_NULL;
    if (misaligned(w_bf16, 16) || misaligned(w_out_bf16, 16) || misaligned(s, 16) ||
        misaligned(gain_inout, 4))
        return QR_ERR_ALIGN;
    const bool inplace = w_out_bf16 == w_bf16;
    const int64_t ld_out = inplace ? ld_w : k;
    const Range rw = span(w_bf16, strided_bytes(n, k, ld_w, 2));
    const Range ro = span(w_out_bf16, strided_bytes(n, k, ld_out, 2));
    const Range rs = span(s, k * 4), rg = span(gain_inout, gain_inout ? k * 4 : 0);
    if ((!inplace && overlap(ro, rw)) || overlap(ro, rs) || overlap(ro, rg) || overlap(rg, rw) ||
        overlap(rg, rs))
        return QR_ERR_ALIAS;
    return launch_status(qr::launch_uaq_fold(static_cast<const uint16_t *>(w_bf16), n, k, ld_w, s,
                                             static_cast<uint16_t *>(w_out_bf16), ld_out,
                                             gain_inout, (hipStream_t)stream));
}

qr_status qr_uaq_fold_quant_w_128x128(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w,
                                       const float *s, void *w_out_bf16, float *gain_inout,
                                       uint8_t *q, float *sq, uint8_t *qT, float *sqT,
                                       qr_stream stream)
{
    const qr_status st = check_weight(w_bf16, n, k, ld_w, q, sq, qT, sqT);
    if (st != QR_OK || n == 0 || k == 0)
        return st;
    if (!s || !w_out_bf16)
        return QR_ERR_NULL;
    if (misaligned(w_out_bf16, 16) || misaligned(s, 16) || misaligned(gain_inout, 4))
        return QR_ERR_ALIGN;
    const bool inplace = w_out_bf16 == w_bf16;
    const int64_t ld_out = inplace ? ld_w : k;
    const int64_t nblk = cdiv(n, 128) * cdiv(k, 128);
    const Range rw = span(w_bf16, strided_bytes(n, k, ld_w, 2)), rs = span(s, k * 4);
    const Range outs[6] = {span(w_out_bf16, strided_bytes(n, k, ld_out, 2)),
                           span(gain_inout, gain_inout ? k * 4 : 0),
                           span(q, n * k), span(sq, nblk * 4), span(qT, n * k),
                           span(sqT, nblk * 4)};
    for (int i = 0; i < 6; ++i) {
        if ((i != 0 || !inplace) && overlap(outs[i], rw))
            return QR_ERR_ALIAS;
        if (overlap(outs[i], rs))
            return QR_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j]))
                return QR_ERR_ALIAS;
    }
    return launch_status(qr::launch_fold_quant_w(static_cast<const uint16_t *>(w_bf16), n, k, ld_w,
                                                 s, static_cast<uint16_t *>(w_out_bf16), ld_out,
                                                 gain_inout, q, sq, qT, sqT,
                                                 (hipStream_t)stream));
}

}  // extern "C"
