/*
 * qr.h -- C ABI of the MI355X (gfx950) fine-grained FP8 quantize-and-multiply library.
 *
 * The library implements the linear-layer hot path that the quantized-rollout RL methods
 * share: 1x128 per-group quantization of activations and gradients, 128x128 per-block
 * quantization of weights, the block-scaled FP8 GEMM in its FProp, DGrad and WGrad forms,
 * and the one-time UAQ invariant-scale fold.
 *
 * Sources (the pages this library follows):
 *   [JET]  "Jet-RL: Enabling On-Policy FP8 Reinforcement Learning with Unified Training and
 *          Rollout Precision Flow" (arXiv 2601.14243v1) paper notes, section "fine-grained GEMM
 *          quantization scheme" (the paper's Figure 6): all three GEMMs of a linear layer run
 *          in FP8; weights are quantized per 128x128 block, activations and gradients per
 *          1x128 group; FProp takes the activation 1x128 row-major and the weight 128x128
 *          "column-major"; DGrad reuses the FProp configuration; WGrad takes its first operand
 *          1x128 and its second 128x1, with the two quantizations fused; gradients travel
 *          between operators in BF16 and are quantized only inside the kernels.  Section
 *          "system implementation": weights are quantized to FP8 in the parameter-update
 *          phase.
 *   [QERL] "QeRL: Beyond Efficiency -- Quantization-enhanced Reinforcement Learning for LLMs"
 *          paper notes (abstract and key takeaways): the rollout runs on NVFP4 weights, a 4-bit
 *          float format with two-level scaling (FP8 E4M3 block scales and an FP32 tensor scale).
 *   [QURL] "QuRL: Efficient Reinforcement Learning with Quantized Rollout" (ICLR 2026) paper
 *          notes, section "key design 1: update-aware quantization (UAQ)": WX = (W/s)(sX) with
 *          s > 1 applied per column of W and per row of the preceding activation, folded into
 *          the norm gain once before RL training.
 *
 * Numeric conventions (the pages say only "FP8"; these are this library's readings):
 *   - FP8 is OCP E4M3: bias 7, largest finite 448, S.1111.111 is NaN, no infinities,
 *     subnormals m*2^-9.  Codes are stored one byte per element.
 *   - A group's scale is s = RN32(amax / 448) (one binary32 division, amax exact).  The code
 *     of x is E4M3(RN32(x / s)), round to nearest even, saturating at +-448, keeping the sign
 *     of zero.  amax == 0 gives s == 0 and signed-zero codes.  A trailing partial group takes
 *     amax over the elements present.
 *   - Dequantized value = code value * group scale.  GEMMs accumulate in fp32 with the scale
 *     product applied once per 128-element contraction group; outputs are fp32 or bf16
 *     (round to nearest even).
 *   - Domain of the FP8 GEMMs' accuracy bound (|y - Y| <= 2e-3 * sum_k |a_k b_k| per output,
 *     Y the exact result): the binary32 product sA * sB of two non-zero group scales that
 *     meet in an output must be at least 2^-126 (binary32's smallest normal), i.e. their
 *     group amax values must multiply to at least about 2^-108.4, and every output and
 *     partial sum must stay below 2^128.  Zero groups (scale 0) are always exact.  Outside
 *     that range the scale product or the output leaves binary32's normal range and the
 *     bound can fail; nothing is reported.  For bf16 inputs it holds whenever every group
 *     amax lies in [2^-54, 2^56] and the outputs fit binary32.
 *   - Inputs must be finite.  Non-finite input is not detected on the GPU; the results are
 *     then undefined, but every access stays in bounds.
 *
 * Conventions of every entry point:
 *   - All tensor pointers are DEVICE pointers, owned and allocated by the caller; the library
 *     allocates nothing and keeps no state between calls.  Tensors are row-major; bf16
 *     tensors are passed as their 16-bit patterns.  Outputs are dense (leading dimension =
 *     their column count); inputs may carry a leading dimension ld (elements).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and the call
 *     returns without synchronizing.  Device faults surface at the caller's next
 *     synchronization, as usual in HIP.
 *   - Arguments are validated on the host before any HIP call; a failed check returns a
 *     status and launches nothing.  A size of zero returns QR_OK and launches nothing.
 *   - Results are bitwise deterministic for a given shape (no atomics on any output path).
 *   - Calls are thread-safe; calls that write the same buffers concurrently race.
 */
#ifndef QR_H
#define QR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qr_status;
enum {
    QR_OK = 0,
    QR_ERR_NULL = 1,        /* a required pointer is NULL, or no output was requested     */
    QR_ERR_SHAPE = 2,       /* negative size, or a size rule of the entry point violated   */
    QR_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                            */
    QR_ERR_ALIAS = 4,       /* an output overlaps an input or another output               */
    QR_ERR_WORKSPACE = 5,   /* workspace smaller than qr_gemm_workspace_bytes() requires   */
    QR_ERR_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch                    */
    QR_ERR_ARG = 7,         /* an enumerated argument is out of range                      */
    QR_ERR_SCRATCH = 8      /* the allocation-free GEMM's scratch is too small for the call  */
};

/* Output element type of the GEMMs.  An int32_t rather than an enum type, so that a caller's
 * out-of-range value reaches the validation (and returns QR_ERR_ARG) without being undefined
 * behaviour in the implementation. */
typedef int32_t qr_out_dtype;
enum { QR_OUT_F32 = 0, QR_OUT_BF16 = 1 };

typedef enum {
    QR_GEMM_FPROP = 0,   /* qr_gemm_fp8_bsfprop   */
    QR_GEMM_DGRAD = 1,   /* qr_gemm_fp8_bsdgrad   */
    QR_GEMM_WGRAD = 2,   /* qr_gemm_fp8_bswgrad   */
    QR_GEMM_INT8 = 3     /* qr_gemm_int8_w8a8     */
} qr_gemm_kind;

typedef void *qr_stream; /* hipStream_t */

/* Human-readable name of a status code (static string, never NULL). */
const char *qr_status_string(qr_status status);

/* Version of this ABI (incremented on any incompatible change). */
int32_t qr_abi_version(void);

/*
 * Activation / gradient quantization [JET].
 *
 * x: bf16 [rows, cols], leading dimension ld_x (elements, >= cols).
 * Row-wise 1x128 groups (128 consecutive elements of a row; FProp's and DGrad's A operand):
 *     q_row [rows, cols] codes, s_row [rows, ceil(cols/128)] fp32 scales.
 * Column-wise 128x1 groups (128 consecutive rows of one column; WGrad's operands), stored
 * transposed so that each group is contiguous:
 *     q_colT [cols, rows] codes, s_colT [cols, ceil(rows/128)] fp32 scales.
 * Either output pair may be NULL (both members NULL), but not both pairs.  Requesting both
 * is the fused quantize-transpose: x is read once.
 *
 * Size rules: rows >= 0, cols >= 0; cols % 8 == 0, ld_x % 8 == 0 and ld_x < 2^22; when the
 * column-wise pair is requested also rows % 8 == 0.  x, q_row, q_colT 16-byte aligned; scale pointers
 * 4-byte aligned.  Outputs must not overlap x or each other.
 */
qr_status qr_quant_act_1x128(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t *q_row, float *s_row, uint8_t *q_colT, float *s_colT,
                             qr_stream stream);

/*
 * 4-bit weights [QERL: QeRL notes, NVFP4 -- 4-bit floats with two-level scaling, FP8 E4M3 block
 * scales and an FP32 tensor scale -- for the rollout's weights].  Readings (the notes give no
 * formula): blocks of 16 consecutive elements along a weight row, and
 *   t = RN32(amax / 2688)                                  (the tensor scale; 2688 = 448 * 6)
 *   bscale[r, b] = E4M3(RN32(amax_b / RN32(6 t)))          (nearest even, saturating)
 *   code = E2M1(RN32(x / RN32(dq(bscale) * t)))            (nearest of 0, .5, 1, 1.5, 2, 3, 4, 6,
 *                                                           ties to even, saturating, signed)
 * A block whose scale encodes to 0 (and an all-zero weight, t == 0) gets signed-zero codes.
 *   w       bf16 [n, k], leading dimension ld_w.
 *   codes   [n, k/2] bytes: element 2j of a row in the low nibble of byte j.
 *   bscale  [n, k/16] E4M3 codes;  tscale: one fp32 (device).
 *   workspace: device scratch of at least QR_NVFP4_WORKSPACE_BYTES; contents do not matter.
 * Size rules: n, k >= 0; k % 32 == 0, ld_w % 8 == 0, ld_w < 2^22.  w and codes 16-byte
 * aligned; no output or the workspace may overlap the input or each other.
 */
#define QR_NVFP4_WORKSPACE_BYTES 4096
qr_status qr_quant_w_nvfp4(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w, uint8_t *codes,
                           uint8_t *bscale, float *tscale, void *workspace,
                           size_t workspace_bytes, qr_stream stream);

/*
 * GEMM of bf16 activations with 4-bit weights (the rollout's decode):
 *   y[m, n] = t * sum_k x[m, k] * E2M1(codes[n, k]) * E4M3(bscale[n, k/16])
 * with the products of x and the dequantized weight (both exact in bf16) accumulated in fp32.
 *   x  bf16 [M, K] dense;  codes / bscale / tscale from qr_quant_w_nvfp4 of W [N, K];
 *   y  [M, N], fp32 or bf16 per y_dtype.
 * Size rules: M, N >= 0, (M + 64) K < 2^31; K % 128 == 0.  x, codes and y 16-byte aligned, bscale
 * 2-byte aligned.
 */
qr_status qr_gemm_w4a16(const void *x_bf16, const uint8_t *codes, const uint8_t *bscale,
                        const float *tscale, int64_t M, int64_t N, int64_t K, void *y,
                        qr_out_dtype y_dtype, qr_stream stream);

/*
 * INT8 W8A8 variant [QURL, experiment setup: channel-wise weight quantization and token-wise
 * activation quantization, INT8 or FP8; the rollout's INT8 GEMM].  Symmetric, one scale per
 * row: a row is a token of an activation or an output channel of a weight [n, k].
 *   s[r] = RN32(amax_r / 127);  q[r, c] = clamp(RNE(RN32(x[r, c] / s[r])), -127, 127)
 * (RNE: nearest integer, ties to even; a row with amax == 0 has s == 0 and zero codes).
 *   x  bf16 [rows, cols], leading dimension ld_x;  q int8 [rows, cols];  s fp32 [rows].
 * Size rules: rows, cols >= 0; cols % 8 == 0, ld_x % 8 == 0, ld_x < 2^22.  x and q 16-byte
 * aligned, s 4-byte aligned; no output may overlap an input or the other output.
 */
qr_status qr_quant_int8_rowwise(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                int8_t *q, float *s, qr_stream stream);

/*
 * INT8 W8A8 GEMM: y[m, n] = sa[m] * sb[n] * sum_k a[m, k] b[n, k], with the integer sum exact
 * (int32) and the scaling in binary32 (y = float(sum) * (sa[m] * sb[n])).
 *   a  int8 [M, K] with sa [M] (qr_quant_int8_rowwise of the activation)
 *   b  int8 [N, K] with sb [N] (qr_quant_int8_rowwise of the weight W[N, K])
 *   y  [M, N], fp32 or bf16 per y_dtype.
 * workspace: device scratch of at least qr_gemm_workspace_bytes(QR_GEMM_INT8, M, N, K) bytes
 *   (may be NULL when that is 0); it then holds the splits' exact int32 partial sums, which
 *   are added before the scaling, so the result is the same as without a split.
 * Size rules: M, N >= 0; K % 128 == 0 and K <= 131072 (the sum stays within int32); with
 * K == 0, a and b may be NULL and y = 0 (for finite scales).  a, b, y, workspace 16-byte
 * aligned, sa, sb 4-byte aligned; neither y nor the workspace may overlap an input or each
 * other.
 */
qr_status qr_gemm_int8_w8a8(const int8_t *a, const float *sa, const int8_t *b, const float *sb,
                            int64_t M, int64_t N, int64_t K, void *y, qr_out_dtype y_dtype,
                            void *workspace, size_t workspace_bytes, qr_stream stream);

/*
 * Norm and activation quantize in one pass (the producer of the FProp operand).  The norm in
 * front of a linear layer carries the UAQ scale in its gain [QURL, key design 1: s is
 * folded into the norm once], and its output is what [JET] quantizes in 1x128 groups; this
 * call does both, so the bf16 activation need not be written and read back:
 *   y[m, c] = RN_bf16((h[m, c] * inv[m]) * gain[c]),  inv[m] = 1 / sqrt(mean_c h[m, c]^2 + eps)
 * (binary32 arithmetic: the sum of squares in one fixed order per row, each operation
 * correctly rounded), then q_row / s_row are y's 1x128 codes and scales exactly as
 * qr_quant_act_1x128 would produce them from y.
 *   h      bf16 [rows, cols], leading dimension ld_h (the hidden state before the norm).
 *   gain   fp32 [cols] (the norm gain, already multiplied by s if the next layer is folded).
 *   eps    >= 0, finite.
 *   y_bf16 NULL, or bf16 [rows, cols] (dense): the normalized activation, for a consumer that
 *          needs it in bf16 (WGrad's 128x1 operand).
 *   q_row [rows, cols] codes, s_row [rows, ceil(cols/128)] scales.
 * Size rules: rows, cols >= 0; cols % 8 == 0, ld_h % 8 == 0, ld_h < 2^22.  h, y, q_row and gain
 * 16-byte aligned, s_row 4-byte aligned.  No output may overlap an input or another output.
 * A bad eps returns QR_ERR_ARG.
 */
qr_status qr_rmsnorm_quant_1x128(const void *h_bf16, int64_t rows, int64_t cols, int64_t ld_h,
                                 const float *gain, float eps, void *y_bf16, uint8_t *q_row,
                                 float *s_row, qr_stream stream);

/*
 * The same norm emitting both activation layouts that training needs [JET, fine-grained GEMM
 * quantization scheme: FProp takes the activation in 1x128 groups and WGrad takes it in 128x1
 * groups, the two quantizations fused; practical advice: the activations kept for the backward
 * pass are FP8].  One call: the row statistics
 *   inv_rms[m] = 1 / sqrt(mean_c h[m, c]^2 + eps)
 * (binary32, the sum of squares in qr_rmsnorm_quant_1x128's order for more than 256 rows), then
 *   y[m, c] = RN_bf16((h[m, c] * inv_rms[m]) * gain[c])
 * and from one read of h, y's 1x128 row codes and scales and its 128x1 column codes and scales
 * stored transposed, exactly as qr_quant_act_1x128 would produce them from y.
 *   h       bf16 [rows, cols], leading dimension ld_h.
 *   gain    fp32 [cols];  eps >= 0, finite.
 *   inv_rms fp32 [rows] out: the statistic above (also what the norm's backward pass needs).
 *   y_bf16  NULL, or bf16 [rows, cols] (dense).
 *   q_row / s_row, q_colT / s_colT: as for qr_quant_act_1x128; either pair may be NULL (both
 *           members), not both.
 * Size rules: rows, cols >= 0; cols % 8 == 0, ld_h % 8 == 0, ld_h < 2^22, ceil(rows/128) <=
 * 65535; rows % 8 == 0 when the column pair is requested.  h, y, q_row, q_colT and gain 16-byte
 * aligned, s_row, s_colT and inv_rms 4-byte aligned.  No output may overlap an input or another
 * output.  A bad eps returns QR_ERR_ARG.  Two launches on `stream`.
 */
qr_status qr_rmsnorm_quant_dual(const void *h_bf16, int64_t rows, int64_t cols, int64_t ld_h,
                                const float *gain, float eps, float *inv_rms, void *y_bf16,
                                uint8_t *q_row, float *s_row, uint8_t *q_colT, float *s_colT,
                                qr_stream stream);

/*
 * Weight quantization, 128x128 blocks [JET]; run once per weight update.
 *
 * w: bf16 [n, k] (n = output features, k = input features), leading dimension ld_w.
 *     q [n, k] codes, s [ceil(n/128), ceil(k/128)] fp32 scales (block (i, j) covers rows
 *     128i.., columns 128j..).
 * Optional transposed copy for DGrad (both NULL or both non-NULL):
 *     qT [k, n] with qT[c, r] = q[r, c], sT [ceil(k/128), ceil(n/128)] with sT[j, i] = s[i, j].
 *
 * Size rules: n, k >= 0; n % 8 == 0, k % 8 == 0, ld_w % 8 == 0, ld_w < 2^22.  Alignment and aliasing as
 * for qr_quant_act_1x128.
 */
qr_status qr_quant_w_128x128(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w,
                             uint8_t *q, float *s, uint8_t *qT, float *sT, qr_stream stream);

/*
 * Weight update re-quantization [JET, section "system implementation": the weights are
 * quantized to FP8 in the parameter-update phase]: every weight of a model is re-quantized
 * after an optimizer step.  This call does a list of them in one launch, with the tiles of
 * all weights shared out over the whole GPU, so small weights do not leave it idle.
 *
 * descs[i] describes one weight exactly as the arguments of qr_quant_w_128x128 (same layouts,
 * size rules and alignment); its qT/sT pair may be NULL for some weights and not others.
 * count: 0 .. QR_MAX_WEIGHT_BATCH; the descriptor array is host memory, read during the call
 * only.  A weight with n == 0 or k == 0 is skipped.
 * Aliasing: no output may overlap any input or any other output, across all descriptors
 * (inputs may overlap each other).  Every descriptor is validated before anything launches;
 * on error nothing runs and the first failing check's status is returned.
 */
typedef struct qr_weight_desc {
    const void *w_bf16;   /* bf16 [n, k], leading dimension ld_w */
    int64_t n, k, ld_w;
    uint8_t *q;           /* [n, k] codes */
    float *s;             /* [ceil(n/128), ceil(k/128)] scales */
    uint8_t *qT;          /* NULL or [k, n] transposed codes */
    float *sT;            /* NULL or [ceil(k/128), ceil(n/128)] transposed scales */
} qr_weight_desc;

#define QR_MAX_WEIGHT_BATCH 4096

qr_status qr_quant_w_128x128_batched(const qr_weight_desc *descs, int32_t count,
                                     qr_stream stream);

/*
 * FProp [JET]:  Y[m, n] = sum_k deq(A)[m, k] * deq(W)[n, k].
 *   a  [M, K] codes with sa [M, K/128]            (1x128 groups along K, from q_row)
 *   b  [N, K] codes with sb [ceil(N/128), K/128]   (the 128x128-quantized weight W[N, K])
 *   y  [M, N], fp32 or bf16 per y_dtype.
 * Size rules: M, N >= 0; K % 128 == 0.  a, b, y 16-byte aligned.
 * workspace: device scratch of at least qr_gemm_workspace_bytes(QR_GEMM_FPROP, M, N, K)
 * bytes (may be NULL when that is 0); its contents on entry do not matter.
 */
qr_status qr_gemm_fp8_bsfprop(const uint8_t *a, const float *sa, const uint8_t *b,
                              const float *sb, int64_t M, int64_t N, int64_t K, void *y,
                              qr_out_dtype y_dtype, void *workspace, size_t workspace_bytes,
                              qr_stream stream);

/*
 * DGrad [JET]:  dX[m, k] = sum_n deq(dY)[m, n] * deq(W)[n, k]  (the FProp form on W^T).
 *   dy  [M, N] codes with sdy [M, N/128]                  (1x128 groups along N, from q_row)
 *   wT  [K, N] codes with swT [ceil(K/128), N/128]        (the transposed copy qT/sT of
 *                                                          qr_quant_w_128x128 for W[N, K])
 *   dx  [M, K], fp32 or bf16.
 * Size rules: M, K >= 0; N % 128 == 0.  Workspace as for FProp (kind QR_GEMM_DGRAD).
 */
qr_status qr_gemm_fp8_bsdgrad(const uint8_t *dy, const float *sdy, const uint8_t *wT,
                              const float *swT, int64_t M, int64_t N, int64_t K, void *dx,
                              qr_out_dtype dx_dtype, void *workspace, size_t workspace_bytes,
                              qr_stream stream);

/*
 * WGrad [JET]:  dW[n, k] = sum_m deq(dY)[m, n] * deq(X)[m, k], contraction over M tokens,
 * both operands grouped 128 along the tokens (dY^T 1x128, X 128x1):
 *   dyT [N, M] codes with sdyT [N, M/128]   (q_colT / s_colT of qr_quant_act_1x128 on dY)
 *   xT  [K, M] codes with sxT  [K, M/128]   (q_colT / s_colT of qr_quant_act_1x128 on X)
 *   dw  [N, K], fp32 or bf16.
 * Size rules: N, K >= 0; M % 128 == 0.  Workspace as for FProp (kind QR_GEMM_WGRAD).
 */
qr_status qr_gemm_fp8_bswgrad(const uint8_t *dyT, const float *sdyT, const uint8_t *xT,
                              const float *sxT, int64_t M, int64_t N, int64_t K, void *dw,
                              qr_out_dtype dw_dtype, void *workspace, size_t workspace_bytes,
                              qr_stream stream);

/*
 * FProp without any allocation: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * size rules, alignment, aliasing and results as qr_gemm_fp8_bsfprop, bit for bit, minus the
 * workspace: where that call would need one (qr_gemm_workspace_bytes(QR_GEMM_FPROP, M, N, K)
 * > 0), the K-split partial sums go to a device scratch array inside the library instead,
 * QR_NOALLOC_SCRATCH_BYTES per GPU, held from the first such call on a GPU until the process
 * ends.  A product whose partial sums do not fit returns QR_ERR_SCRATCH and launches nothing.
 * The call allocates nothing and calls no allocating routine.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in time on one GPU
 * (other streams, other threads) race and must be serialized by the caller; calls on one
 * stream are ordered and safe.  The scratch keeps the last call's partial sums; every call
 * writes all of the partial sums it reads, so nothing needs clearing.
 */
#define QR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
qr_status qr_gemm_fp8_bsfprop_noalloc(const uint8_t *a, const float *sa, const uint8_t *b,
                                      const float *sb, int64_t M, int64_t N, int64_t K, void *y,
                                      qr_out_dtype y_dtype, qr_stream stream);

/* Workspace bytes the GEMM entry point of `kind` needs for these sizes (0 if none).  The
 * sizes are the ones passed to that entry point.  Returns 0 for invalid arguments.
 * It is non-zero when the product is split over its contraction to occupy the GPU: up to
 * 256 output rows (decode batches) against a narrow weight, or few 256x256 output tiles.  The
 * splits' partial sums [split][rows][cols] (fp32; int32 for QR_GEMM_INT8) are then added in
 * split order, so results do not depend on timing. */
size_t qr_gemm_workspace_bytes(int32_t kind, int64_t M, int64_t N, int64_t K);

/*
 * UAQ fold [QURL]:  w_out[n, c] = RN_bf16(w[n, c] / s[c])  (the exact quotient rounded once
 * to bf16, nearest even) and, if gain_inout != NULL, gain_inout[c] = RN32(gain_inout[c] * s[c]).
 *   w      bf16 [n, k], leading dimension ld_w; w_out may equal w (in place, same ld_w),
 *          otherwise w_out is dense [n, k] and must not overlap w.
 *   s      fp32 [k], every s[c] finite and > 0 (not checked on the GPU).
 *   gain   fp32 [k] or NULL: the gain of the norm that feeds this layer.
 * Run once, before training; the fold is NOT idempotent (a second call divides by s again).
 * Size rules: n, k >= 0; k % 8 == 0, ld_w % 8 == 0; w, w_out and s 16-byte aligned, gain_inout
 * 4-byte aligned.  w_out must not overlap s or gain_inout, nor gain_inout w or s.
 */
qr_status qr_uaq_fold(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w, const float *s,
                      void *w_out_bf16, float *gain_inout, qr_stream stream);

/*
 * UAQ fold followed by the 128x128 weight quantization, in one pass over w [QURL, key design
 * 1: s folded into the weights once; JET, fine-grained GEMM quantization scheme: 128x128
 * weight blocks].
 * The outputs equal those of qr_uaq_fold(w, n, k, ld_w, s, w_out, gain_inout) followed by
 * qr_quant_w_128x128(w_out, n, k, ld_out, q, sq, qT, sqT), bit for bit, where ld_out is ld_w
 * in place and k otherwise; w is read once and the folded weight is not read back.
 *   w, s, w_out, gain_inout as for qr_uaq_fold; q, sq, qT, sqT as for qr_quant_w_128x128.
 * Size rules: those of both entry points (n % 8 == 0, k % 8 == 0, ld_w % 8 == 0, ld_w >= k,
 * ld_w < 2^22, ceil(n/128) <= 65535).  Alignment: w, w_out, s, q, qT 16 bytes; sq, sqT,
 * gain_inout 4 bytes.  No output may overlap w (except w_out in place), s or another output.
 */
qr_status qr_uaq_fold_quant_w_128x128(const void *w_bf16, int64_t n, int64_t k, int64_t ld_w,
                                       const float *s, void *w_out_bf16, float *gain_inout,
                                       uint8_t *q, float *sq, uint8_t *qT, float *sqT,
                                       qr_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QR_H */
