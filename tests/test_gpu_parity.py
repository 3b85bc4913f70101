"""GPU parity: the HIP library through its C ABI against the reference oracle.

Codes and scales must match bit for bit; GEMM outputs must satisfy
|gpu - oracle| <= 2e-3 * sum_k |a_k b_k| per element against the unrounded fp64 oracle.
Every output is compared in full, at the named workloads' full sizes too (there with the bare
2e-3 bound, no allowance for the bf16 output rounding); a few extra shapes are sampled.
Quantizer and GEMM outputs sit between guard bands whose pattern must survive each call.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_qr_amd as qr
import oracle
import qr_synth
from gpu_util import (assert_bitexact, assert_gemm_close, check_norm_y, check_w4a16, dev,
                      dev_bf16, g_gemm_dgrad, g_gemm_fprop, g_gemm_wgrad, g_quant_act, g_quant_w,
                      host, out_f64, sample_positions)

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qr.load()


def say(*a):
    print("[case]", *a, flush=True)


# ================================================================= quantizers

ACT_SHAPES = [(256, 512, "tiny_fprop X"), (77, 200, "ragged rows and partial group"),
              (1, 8, "one row, 8 columns"), (300, 1096, "ragged both"),
              (8192, 4096, "prefill_8b X full size")]


@pytest.mark.parametrize("rows,cols,name", ACT_SHAPES)
def test_quant_rows(rows, cols, name):
    say("quant_rows", rows, cols, name)
    x = qr_synth.normal_bf16(rows * 7 + cols, (rows, cols), 1.0, 99, max(1, cols // 100))
    q, s, _, _ = g_quant_act(qr, dev_bf16(x), row=True, col=False)
    rq, rs = oracle.quant_rows(x)
    assert_bitexact(host(q), rq, "codes")
    assert_bitexact(host(s), rs, "scales")


DUAL_SHAPES = [(256, 512, "small"), (200, 136, "ragged rows and columns"), (8, 8, "minimal"),
               (264, 392, "rows % 16 == 8 over several tiles"),
               (8192, 4096, "backward_8b dY full size")]


@pytest.mark.parametrize("rows,cols,name", DUAL_SHAPES)
def test_quant_dual_and_colT(rows, cols, name):
    say("quant dual", rows, cols, name)
    std = 1e-3 if rows == 8192 else 1.0
    x = (qr_synth.backward_8b_dy() if rows == 8192 else
         qr_synth.normal_bf16(rows + cols, (rows, cols), std, 5, 2))
    xd = dev_bf16(x)
    q, s, qT, sT = g_quant_act(qr, xd, row=True, col=True)
    rq, rs = oracle.quant_rows(x)
    rqT, rsT = oracle.quant_cols_T(x)
    assert_bitexact(host(q), rq, "row codes")
    assert_bitexact(host(s), rs, "row scales")
    assert_bitexact(host(qT), rqT, "colT codes")
    assert_bitexact(host(sT), rsT, "colT scales")
    # column-only pass (X's WGrad operand) gives the same column outputs
    _, _, qT2, sT2 = g_quant_act(qr, xd, row=False, col=True)
    assert_bitexact(host(qT2), rqT, "colT-only codes")
    assert_bitexact(host(sT2), rsT, "colT-only scales")


W_SHAPES = [(512, 512, "tiny_fprop W"), (200, 136, "ragged blocks"),
            (392, 264, "n % 16 == 8 over several blocks"),
            (4096, 4096, "prefill_8b W"), (14336, 4096, "decode_8b W")]


@pytest.mark.parametrize("n,k,name", W_SHAPES)
def test_quant_w(n, k, name):
    say("quant_w", n, k, name)
    w = qr_synth.normal_bf16(n + 3 * k, (n, k), 0.02)
    q, s, qT, sT = g_quant_w(qr, dev_bf16(w), transposed=True)
    rq, rs = oracle.quant_blocks(w)
    assert_bitexact(host(q), rq, "codes")
    assert_bitexact(host(s), rs, "scales")
    assert_bitexact(host(qT), np.ascontiguousarray(rq.T), "transposed codes")
    assert_bitexact(host(sT), np.ascontiguousarray(rs.T), "transposed scales")


def test_quant_w_batched():
    """A weight update's re-quantization in one call: 41 descriptors (more than one launch
    table of 32), ragged and 8B-sized shapes, the transposed copy for some and not others, a
    strided input, two descriptors sharing one input, and an empty weight (skipped)."""
    say("quant_w batched")
    rng = np.random.default_rng(17)
    small = [(200, 136), (392, 264), (128, 128), (8, 8), (136, 8), (8, 392), (256, 520)]
    shapes = [small[i % len(small)] for i in range(36)] + [(4096, 4096), (1024, 4096)]
    hosts = [qr_synth.normal_bf16(900 + i, sh, float(rng.uniform(0.005, 0.05)))
             for i, sh in enumerate(shapes)]
    ws = [dev_bf16(h) for h in hosts]
    flags = [bool(i % 3) for i in range(len(ws))]
    big = qr_synth.normal_bf16(950, (256, 640), 0.02)           # strided: ld 640, k 384
    hosts.append(np.ascontiguousarray(big[:, 64:448]))
    ws.append(dev_bf16(big)[:, 64:448])
    flags.append(True)
    hosts.append(hosts[2])                                      # same input, second descriptor
    ws.append(ws[2])
    flags.append(not flags[2])
    outs = qr.quant_w_batched(ws, flags)
    # an empty weight among real ones: its (unused) pointers may be anything non-null
    q0, s0, _, _ = outs[0]
    items = [(ws[3], 0, 8, 8, q0, s0, None, None)]
    for w, (q, s, qT, sT) in zip(ws, outs):
        items.append((w, w.shape[0], w.shape[1], w.stride(0), q, s, qT, sT))
    assert len(items) == 41
    qr.qr_quant_w_128x128_batched(items)
    for i, (h, (q, s, qT, sT)) in enumerate(zip(hosts, outs)):
        rq, rs = oracle.quant_blocks(h)
        assert_bitexact(host(q), rq, f"codes {i}")
        assert_bitexact(host(s), rs, f"scales {i}")
        if flags[i]:
            assert_bitexact(host(qT), np.ascontiguousarray(rq.T), f"transposed codes {i}")
            assert_bitexact(host(sT), np.ascontiguousarray(rs.T), f"transposed scales {i}")
        else:
            assert qT is None and sT is None


RMS_SHAPES = [(256, 512, 1e-6, "small"), (77, 200, 1e-6, "ragged rows, partial group"),
              (1, 8, 1e-5, "one row, 8 columns"), (300, 5120, 1e-6, "32B hidden: 10 passes"),
              (40, 27648, 1e-6, "down-proj width: row read twice"),
              (8192, 4096, 1e-6, "prefill_8b hidden full size"),
              (333, 4096, 1e-5, "whole 512-column passes, rows % 4 != 0"),
              # few rows: a workgroup of 8 waves per row (one pass each, several passes kept
              # in registers, and the re-read path), ragged columns
              (64, 4096, 1e-6, "decode_8b hidden, 8 waves per row"),
              (256, 5120, 1e-6, "32B decode hidden, passes in registers"),
              (3, 1096, 1e-5, "few rows, ragged columns"),
              (16, 70000, 1e-6, "few rows, row read twice")]


@pytest.mark.parametrize("rows,cols,eps,name", RMS_SHAPES)
def test_rmsnorm_quant(rows, cols, eps, name):
    """The fused norm + 1x128 quantize.  y is RN_bf16 of a binary32 evaluation whose sum of
    squares has a relative error below ~2^-18, so y may differ from RN_bf16(exact) by one
    ulp only where the exact value lies within 2^-17 (relative) of a bf16 midpoint; the
    codes and scales must equal the oracle's 1x128 quantizer applied to the GPU's y, and the
    call without y must give the same codes."""
    say("rmsnorm_quant", rows, cols, name)
    rng = np.random.default_rng(rows + cols)
    h = qr_synth.normal_bf16(rows * 3 + cols, (rows, cols), 1.0, 7, max(1, cols // 100))
    s_uaq = rng.uniform(1.5, 4.0, cols).astype(np.float32)      # gain carrying a UAQ scale
    g = (rng.uniform(0.5, 2.0, cols) * s_uaq).astype(np.float32)
    if rows > 4:
        h[1] = 0                                                  # a zero row (eps > 0)
        h[2] = qr_synth.f32_to_bf16_bits(np.full(cols, 3.0e-39, np.float32))  # subnormals
    if cols >= 256:
        g[128:256] *= np.float32(1e-39)     # a group whose y values are all subnormal
    hd, gd = dev_bf16(h), dev(g)
    y, q, s = qr.rmsnorm_quant(hd, gd, eps)
    yg = host(y)
    check_norm_y(yg, h, g, eps)
    rq, rs = oracle.quant_rows(np.ascontiguousarray(yg))
    assert_bitexact(host(q), rq, "codes of y")
    assert_bitexact(host(s), rs, "scales of y")
    _, q2, s2 = qr.rmsnorm_quant(hd, gd, eps, want_y=False)
    assert_bitexact(host(q2), host(q), "codes without y")
    assert_bitexact(host(s2), host(s), "scales without y")


NORM_DUAL_SHAPES = [(256, 512, 1e-6, "small"), (200, 136, 1e-6, "ragged rows and columns"),
                    (8, 8, 1e-5, "minimal"), (264, 392, 1e-6, "rows % 16 == 8, several tiles"),
                    (64, 27648, 1e-6, "wide rows"), (8192, 4096, 1e-6, "prefill_8b hidden")]


@pytest.mark.parametrize("rows,cols,eps,name", NORM_DUAL_SHAPES)
def test_rmsnorm_quant_dual(rows, cols, eps, name):
    """The norm emitting both layouts: inv_rms within the binary32 evaluation's bound of the
    fp64 statistic; y as the single-layout norm's rule; the 1x128 rows and the transposed
    128x1 columns bit-exact against the oracle's quantizers applied to the GPU's y; the same
    codes without y and with one pair only; for more than 256 rows the single-layout entry
    point's y and codes are reproduced bit for bit (same summation order)."""
    say("rmsnorm_quant_dual", rows, cols, name)
    rng = np.random.default_rng(rows * 5 + cols)
    h = qr_synth.normal_bf16(rows * 11 + cols, (rows, cols), 1.0, 9, max(1, cols // 100))
    g = (rng.uniform(0.5, 2.0, cols) * rng.uniform(1.5, 4.0, cols)).astype(np.float32)
    if rows > 4:
        h[1] = 0                                                  # a zero row (eps > 0)
        h[2] = qr_synth.f32_to_bf16_bits(np.full(cols, 3.0e-39, np.float32))  # subnormals
    if cols >= 256:
        g[128:256] *= np.float32(1e-39)     # a group whose y values are all subnormal
    hd, gd = dev_bf16(h), dev(g)
    inv, y, q, s, qT, sT = qr.rmsnorm_quant_dual(hd, gd, eps, want_y=True)
    hf = qr_synth.bf16_bits_to_f32(h).astype(np.float64)
    inv64 = 1.0 / np.sqrt((hf * hf).mean(axis=1) + float(np.float32(eps)))
    invg = host(inv).astype(np.float64)
    assert np.all(np.abs(invg - inv64) <= 2.0 ** -18 * inv64), float(np.max(np.abs(invg / inv64 - 1)))
    yg = host(y)
    check_norm_y(yg, h, g, eps)
    rq, rs = oracle.quant_rows(np.ascontiguousarray(yg))
    rqT, rsT = oracle.quant_cols_T(np.ascontiguousarray(yg))
    assert_bitexact(host(q), rq, "row codes of y")
    assert_bitexact(host(s), rs, "row scales of y")
    assert_bitexact(host(qT), rqT, "colT codes of y")
    assert_bitexact(host(sT), rsT, "colT scales of y")
    _, _, q2, s2, qT2, sT2 = qr.rmsnorm_quant_dual(hd, gd, eps, want_y=False)
    assert_bitexact(host(q2), rq, "row codes without y")
    assert_bitexact(host(qT2), rqT, "colT codes without y")
    _, _, q3, s3, _, _ = qr.rmsnorm_quant_dual(hd, gd, eps, col=False)
    assert_bitexact(host(q3), rq, "row pair only")
    _, _, _, _, qT4, sT4 = qr.rmsnorm_quant_dual(hd, gd, eps, row=False)
    assert_bitexact(host(sT4), rsT, "column pair only")
    if rows > 256:
        y1, q1, s1 = qr.rmsnorm_quant(hd, gd, eps)
        assert_bitexact(host(y1), yg, "y of the single-layout entry point")
        assert_bitexact(host(q1), host(q), "row codes of the single-layout entry point")


INT8_ROWS = [(256, 512), (77, 200), (1, 8), (300, 5120), (40, 27648), (8192, 4096)]


@pytest.mark.parametrize("rows,cols", INT8_ROWS)
def test_quant_int8_rows(rows, cols):
    """One symmetric INT8 scale per row: codes and scales bit-exact.  Covers the register-
    resident rows (up to 8192 columns) and re-read rows, partial passes, a zero row, a row of
    bf16 subnormals (a lifted scale) and a row of huge values."""
    say("quant_int8", rows, cols)
    x = qr_synth.normal_bf16(rows * 5 + cols, (rows, cols), 1.0, 11, max(1, cols // 100))
    if rows > 4:
        x[1] = 0
        x[2] = qr_synth.f32_to_bf16_bits(np.linspace(-3e-39, 3e-39, cols).astype(np.float32))
        x[3] = qr_synth.f32_to_bf16_bits(np.linspace(-3e38, 2e38, cols).astype(np.float32))
    q, s = qr.quant_int8(dev_bf16(x))
    rq, rs = oracle.quant_int8_rows(x)
    assert_bitexact(host(q), rq, "int8 codes")
    assert_bitexact(host(s), rs, "int8 scales")


def _int8_case(M, N, K, seed):
    x = qr_synth.normal_bf16(seed, (M, K), 1.0, seed + 1, max(1, K // 100))
    w = qr_synth.normal_bf16(seed + 2, (N, K), 0.02)
    qa, sa = oracle.quant_int8_rows(x)
    qb, sb = oracle.quant_int8_rows(w)
    return qa, sa, qb, sb


def _check_int8(y, Y, out):
    """fp32 out: |y - Y| <= 2^-22 |Y| (three binary32 roundings in the epilogue); bf16 out:
    plus the bf16 rounding, at most 2^-8 |Y| (8 significant bits)."""
    rel = 2.0 ** -22 if out == qr.QR_OUT_F32 else 2.0 ** -8 + 2.0 ** -21
    err = np.abs(y - Y)
    assert np.all(err <= rel * np.abs(Y)), float(np.max(err / np.maximum(np.abs(Y), 1e-300)))


def _int8_scaled_exact(qa, sa, qb, sb):
    """The entry point's definition in binary32: float(exact integer sum) * (sa[m] * sb[n]).
    The integer sums are formed in binary64, exact because every partial sum is an integer of
    magnitude at most K * 127^2 < 2^53."""
    assert qa.shape[1] * 127 * 127 < 2 ** 53
    S = qa.astype(np.float64) @ qb.astype(np.float64).T
    assert np.abs(S).max(initial=0) < 2 ** 31
    scale = sa.astype(np.float32)[:, None] * sb.astype(np.float32)[None, :]
    return S.astype(np.float32) * scale


# Small products (their K walks on 256-row tiles would be short) take the 64x64 tiles: most of
# the shapes below, (64, 512, 4096) and (40, 1000, 2304) split 4 and 2 ways, and (130, 201, 2048)
# an odd N on a 2-way split (scalar partial stores and sums).  (2050, 4104, 128) and
# (2050, 4100, 128): unsplit 256x256 tiles with ragged M and N, the bf16 output staged through
# LDS (N % 8 == 0) and stored directly (N % 8 != 0).
@pytest.mark.parametrize("M,N,K", [(77, 200, 384), (64, 1000, 1024), (1, 128, 128),
                                   (300, 264, 256), (520, 304, 384), (17, 72, 640),
                                   (64, 512, 4096), (40, 1000, 2304), (130, 201, 512),
                                   (130, 201, 2048), (2050, 4104, 128), (2050, 4100, 128),
                                   (520, 264, 128), (520, 300, 128)])
@pytest.mark.parametrize("out", [qr.QR_OUT_F32, qr.QR_OUT_BF16])
def test_gemm_int8(M, N, K, out):
    say("gemm_int8", M, N, K, out)
    qa, sa, qb, sb = _int8_case(M, N, K, M + N + K)
    y = qr.gemm_int8(dev(qa), dev(sa), dev(qb), dev(sb), out_dtype=out)
    _check_int8(out_f64(y), oracle.gemm_int8(qa, sa, qb, sb), out)
    if out == qr.QR_OUT_F32:
        # split or not, the integer sum is exact and scaled once: equal bits
        assert np.array_equal(y.cpu().numpy(), _int8_scaled_exact(qa, sa, qb, sb))


def test_gemm_int8_multi_band_split_exact():
    """256x256 tiles over three row bands with K split 10 ways (7 groups per split, the last
    one shorter): bit-exact fp32 against float(exact sum) * (sa * sb)."""
    M, N, K = 520, 2048, 8192
    say("gemm_int8 multi-band split", M, N, K)
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, M, N, K) == 10 * M * N * 4
    qa, sa, qb, sb = _int8_case(M, N, K, 31)
    y = qr.gemm_int8(dev(qa), dev(sa), dev(qb), dev(sb), out_dtype=qr.QR_OUT_F32)
    assert np.array_equal(host(y), _int8_scaled_exact(qa, sa, qb, sb))


def test_gemm_int8_empty_zero_k_and_workspace_reuse():
    """K = 0 stores zeros, M = 0 is a no-op; then one workspace serves a split product and a
    smaller split product after it (every partial is rewritten by each call, so nothing of the
    first call leaks into the second)."""
    say("gemm_int8 empty / K=0 / workspace reuse")
    a = torch.zeros((4, 0), dtype=torch.int8, device="cuda")
    y = torch.full((4, 8), 7.0, device="cuda")
    qr.qr_gemm_int8_w8a8(a, torch.ones(4, device="cuda"), a, torch.ones(8, device="cuda"),
                         4, 8, 0, y, qr.QR_OUT_F32)
    assert float(y.abs().max()) == 0.0
    qr.qr_gemm_int8_w8a8(None, None, None, None, 0, 8, 128, y, qr.QR_OUT_F32)   # M = 0
    shapes = [(200, 5888, 5120), (100, 136, 2048)]   # 256x128 tiles split 5 ways; 64x64 split 2
    nb = max(qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, *sh) for sh in shapes)
    assert all(qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, *sh) > 0 for sh in shapes)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for M, N, K in shapes:
        qa, sa, qb, sb = _int8_case(M, N, K, 7 * M + N)
        yd = torch.empty((M, N), dtype=torch.float32, device="cuda")
        qr.qr_gemm_int8_w8a8(dev(qa), dev(sa), dev(qb), dev(sb), M, N, K, yd, qr.QR_OUT_F32,
                             ws, nb)
        assert np.array_equal(yd.cpu().numpy(), _int8_scaled_exact(qa, sa, qb, sb))
        _check_int8(out_f64(yd), oracle.gemm_int8(qa, sa, qb, sb), qr.QR_OUT_F32)


@pytest.mark.parametrize("M,N,K", [(8192, 4096, 4096), (64, 14336, 4096), (256, 5120, 27648),
                                   (256, 55296, 5120), (200, 32768, 256), (256, 7168, 5120),
                                   (64, 4096, 14336)])
def test_gemm_int8_full_size(M, N, K):
    """The 8B prefill shape, the 8B decode shape, the 32B down (K split 12 ways) and gate+up
    projections at batch 256, a ragged-M batch with two K groups on 256 unsplit 256x128 tiles,
    the 32B QKV at batch 256 (256x128 tiles, split 4 ways) and the 8B down at batch 64 (64x64
    tiles, split 4 ways); every output."""
    say("gemm_int8 full", M, N, K)
    qa, sa, qb, sb = _int8_case(M, N, K, 3 * M + N)
    y = out_f64(qr.gemm_int8(dev(qa), dev(sa), dev(qb), dev(sb), out_dtype=qr.QR_OUT_BF16))
    Y = oracle.gemm_int8(qa, sa, qb, sb)
    _check_int8(y, Y, qr.QR_OUT_BF16)


FP4_W = [(64, 128), (200, 96), (1, 32), (4096, 4096), (14336, 4096)]


@pytest.mark.parametrize("n,k", FP4_W)
def test_quant_nvfp4(n, k):
    """4-bit weights: codes, block scales and the tensor scale bit-exact, including an all-zero
    row, a block far below the tensor's amax (its scale encodes to 0: signed-zero codes), one with
    a subnormal block scale and the amax element (scale 448, code 6)."""
    say("quant_nvfp4", n, k)
    w = qr_synth.normal_bf16(n * 3 + k, (n, k), 0.02)
    if n > 2:
        w[1] = 0
        w[2, :16] = qr_synth.f32_to_bf16_bits(np.full(16, -1e-12, np.float32))
        # a block whose E4M3 scale is subnormal (about 0.0068 of the tensor unit)
        w[2, 16:32] = qr_synth.f32_to_bf16_bits(
            np.linspace(-7.6e-6, 7.6e-6, 16).astype(np.float32))
        w[0, 5] = qr_synth.f32_to_bf16_bits(np.array([0.5], np.float32))[0]
    codes, bs, t = qr.quant_nvfp4(dev_bf16(w))
    rc, rb, rt = oracle.quant_nvfp4(w)
    assert_bitexact(host(bs), rb, "block scales")
    assert_bitexact(host(codes), rc, "codes")
    assert_bitexact(host(t), np.array([rt], np.float32), "tensor scale")


def test_quant_nvfp4_midpoint_quotients():
    """Quotients x / e exactly on the E2M1 midpoints (ties to the even code), exactly on E2M1
    values, and one bf16 step either side of them: the tensor amax 2.625 makes t = 2^-10 and
    each block's amax 6 c t makes its scale code the E4M3 value c, so e = c t and every x = m e
    is exact in bf16.  Exact quotients take the kernel's division path, their neighbours the
    reciprocal path; both must match the oracle bit for bit."""
    say("quant_nvfp4 midpoint quotients")
    f32 = np.float32
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    vals = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    cs = [448.0, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 0.5, 0.625, 0.875, 6.0, 10.0, 13.0,
          104.0, 0.1875, 28.0, 52.0, 240.0]
    rows = []
    for b, c in enumerate(cs):
        e = c * 2.0 ** -10
        for variant in range(4):
            x = np.empty(16)
            x[0] = 6.0 * e                                   # the block amax: code 6 (7)
            base = mids if variant % 2 == 0 else vals
            x[1:8] = base * e
            x[8:15] = -base * e
            x[15] = 2.5 * e
            xb = qr_synth.f32_to_bf16_bits(x.astype(f32))
            if variant >= 2:   # one bf16 step up or down from each (amax elements kept)
                step = np.where(np.arange(16) % 2 == 0, 1, -1).astype(np.int32)
                step[np.abs(x) == 6.0 * e] = 0   # the block amax stays the largest magnitude
                mag = (xb & 0x7FFF).astype(np.int32) + step * (1 if variant == 2 else -1)
                xb = ((xb & 0x8000) | np.clip(mag, 0, 0x7F7F)).astype(np.uint16)
            rows.append(xb)
    w = np.concatenate(rows).reshape(-1, 256)
    codes, bs, t = qr.quant_nvfp4(dev_bf16(w))
    rc, rb, rt = oracle.quant_nvfp4(w)
    assert rt == 2.0 ** -10
    assert_bitexact(host(bs), rb, "block scales")
    assert_bitexact(host(codes), rc, "codes")
    assert_bitexact(host(t), np.array([rt], np.float32), "tensor scale")


def test_quant_nvfp4_strided_and_zero():
    say("quant_nvfp4 strided, zero")
    big = qr_synth.normal_bf16(13, (96, 640), 0.02)
    codes, bs, t = qr.quant_nvfp4(dev_bf16(big)[:, 64:448])      # ld 640, k 384
    rc, rb, rt = oracle.quant_nvfp4(np.ascontiguousarray(big[:, 64:448]))
    assert_bitexact(host(codes), rc, "codes")
    assert_bitexact(host(bs), rb, "block scales")
    z = np.zeros((8, 64), np.uint16)
    z[3, 7] = 0x8000
    codes, bs, t = qr.quant_nvfp4(dev_bf16(z))
    rc, rb, rt = oracle.quant_nvfp4(z)
    assert_bitexact(host(codes), rc, "zero codes")
    assert host(t)[0] == 0.0 and not host(bs).any()


@pytest.mark.parametrize("M,N,K", [(64, 1000, 1024), (17, 72, 640), (1, 128, 128),
                                   (100, 264, 256), (200, 520, 384),
                                   # decode batches: ragged N with K steps that do not divide
                                   # among the four waves, long K, N % 4 != 0
                                   (33, 1000, 4608), (5, 72, 8192), (64, 264, 2176),
                                   (7, 13, 4608), (7, 13, 2304)])
def test_gemm_w4a16(M, N, K):
    say("gemm_w4a16", M, N, K)
    x = qr_synth.normal_bf16(M + N + K, (M, K), 1.0, 3, max(1, K // 100))
    w = qr_synth.normal_bf16(M * N + K, (N, K), 0.02)
    codes, bs, t = qr.quant_nvfp4(dev_bf16(w))
    hc, hb, ht = host(codes), host(bs), float(host(t)[0])
    y = out_f64(qr.gemm_w4a16(dev_bf16(x), codes, bs, t, out_dtype=qr.QR_OUT_F32))
    Y = oracle.gemm_w4a16(x, hc, hb, ht)
    absw = oracle.gemm_w4a16(x & np.uint16(0x7FFF), hc & np.uint8(0x77), hb, ht)  # sum |x w| t
    check_w4a16(y, Y, K * 2.0 ** -23 * np.abs(absw))


@pytest.mark.parametrize("M,N,K", [(64, 14336, 4096), (256, 5120, 27648)])
def test_gemm_w4a16_full_size_sampled(M, N, K):
    say("gemm_w4a16 full", M, N, K)
    x = qr_synth.normal_bf16(M + 7, (M, K), 1.0, 9, max(1, K // 100))
    w = qr_synth.normal_bf16(N + 11, (N, K), 0.02)
    codes, bs, t = qr.quant_nvfp4(dev_bf16(w))
    hc, hb, ht = host(codes), host(bs), float(host(t)[0])
    y = out_f64(qr.gemm_w4a16(dev_bf16(x), codes, bs, t, out_dtype=qr.QR_OUT_BF16))
    mi, ni = sample_positions(M, N, 2048, seed=M + N)
    Y = oracle.gemm_w4a16(x, hc, hb, ht, sample=(mi, ni))
    absw = oracle.gemm_w4a16(x & np.uint16(0x7FFF), hc & np.uint8(0x77), hb, ht, sample=(mi, ni))
    check_w4a16(y[mi, ni], Y, K * 2.0 ** -23 * np.abs(absw))


def test_quant_strided_input():
    say("quant strided ld")
    big = qr_synth.normal_bf16(11, (96, 640), 1.0)
    xd = dev_bf16(big)[:, 64:64 + 384]          # ld = 640, cols = 384
    q, s, qT, sT = g_quant_act(qr, xd, row=True, col=True)
    sub = np.ascontiguousarray(big[:, 64:448])
    rq, rs = oracle.quant_rows(sub)
    rqT, rsT = oracle.quant_cols_T(sub)
    assert_bitexact(host(q), rq, "codes")
    assert_bitexact(host(s), rs, "scales")
    assert_bitexact(host(qT), rqT, "colT codes")
    assert_bitexact(host(sT), rsT, "colT scales")
    # rows only: 96 rows take the few-rows kernel (one wave per 512-column slice; the slice
    # holds 3 of its 4 groups here)
    q1, s1, _, _ = g_quant_act(qr, xd, row=True, col=False)
    assert_bitexact(host(q1), rq, "codes, few-rows kernel")
    assert_bitexact(host(s1), rs, "scales, few-rows kernel")


def _groups_for_amax(amax_bits_list):
    """Rows of 128 bf16: first element the group amax, then every bf16 x with |x| <= amax."""
    allb = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    allv = qr_synth.bf16_bits_to_f32(allb)
    finite = np.isfinite(allv)
    rows = []
    for ab in amax_bits_list:
        a = qr_synth.bf16_bits_to_f32(np.array([ab], np.uint16))[0]
        xs = allb[finite & (np.abs(allv) <= a)]
        pad = (-xs.size) % 127
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        r = np.empty((xs.shape[0], 128), np.uint16)
        r[:, 0] = ab
        r[:, 1:] = xs
        rows.append(r)
    return np.concatenate(rows)


def test_codes_every_bf16_for_sampled_scales():
    """Every bf16 x against 1/97 of all finite bf16 amax values (subnormal, normal, huge) and
    hand-picked ones: exercises the exact quotient, saturation, the sign of zero and every
    E4M3 rounding boundary of the hardware conversion."""
    say("exhaustive-x codes")
    picks = list(range(1, 0x7F80, 97)) + [0x0001, 0x0080, 0x3F80, 0x43E0, 0x7F7F, 0x3B12]
    x = _groups_for_amax(np.array(picks, np.uint16))
    for r0 in range(0, x.shape[0], 1 << 19):
        part = np.ascontiguousarray(x[r0:r0 + (1 << 19)])
        q, s, _, _ = g_quant_act(qr, dev_bf16(part), row=True)
        rq, rs = oracle.quant_rows(part)
        assert_bitexact(host(s), rs, "scales")
        assert_bitexact(host(q), rq, "codes")


def test_quant_special_values():
    say("special values")
    x = np.zeros((16, 256), np.uint16)
    x[1, :] = 0x8000                                   # all negative zero
    x[2, :128] = 0x3F80                                # all equal
    x[3, 5] = 0x0001                                   # subnormal amax, rest zero
    x[3, 6] = 0x8001
    x[4, :] = qr_synth.f32_to_bf16_bits(np.linspace(-448, 448, 256).astype(np.float32))
    x[5, :] = qr_synth.f32_to_bf16_bits(np.full(256, 3.0e38, np.float32))
    x[6, ::2] = 0x7F7F                                 # max finite bf16 and its negative
    x[6, 1::2] = 0xFF7F
    x[7, :] = qr_synth.f32_to_bf16_bits((np.arange(256) - 128).astype(np.float32) * 2.0 ** -130)
    q, s, qT, sT = g_quant_act(qr, dev_bf16(x), row=True, col=True)
    rq, rs = oracle.quant_rows(x)
    rqT, rsT = oracle.quant_cols_T(x)
    assert_bitexact(host(q), rq, "codes")
    assert_bitexact(host(s), rs, "scales")
    assert_bitexact(host(qT), rqT, "colT codes")
    assert_bitexact(host(sT), rsT, "colT scales")
    # rows only (16 rows: the few-rows kernel, incl. its lifted quotient for tiny scales)
    q1, s1, _, _ = g_quant_act(qr, dev_bf16(x), row=True, col=False)
    assert_bitexact(host(q1), rq, "codes, few-rows kernel")
    assert_bitexact(host(s1), rs, "scales, few-rows kernel")
    w = np.ascontiguousarray(np.tile(x, (8, 1))[:128])
    qw, sw, _, _ = g_quant_w(qr, dev_bf16(w))
    rqw, rsw = oracle.quant_blocks(w)
    assert_bitexact(host(qw), rqw, "block codes")
    assert_bitexact(host(sw), rsw, "block scales")


# ================================================================= UAQ fold

def test_uaq_fold_random_and_near_midpoints():
    say("uaq fold")
    rng = np.random.default_rng(5)
    w = qr_synth.normal_bf16(61, (64, 256), 0.02)
    s = rng.uniform(1.5, 4.0, 256).astype(np.float32)
    # near-midpoint scales: s = RN32(|w| / mid) for a bf16 midpoint below |w| / 1.5
    wv = qr_synth.bf16_bits_to_f32(w[0]).astype(np.float64)
    for c in range(0, 256, 2):
        tgt = abs(wv[c]) / rng.uniform(1.5, 4.0)
        e = np.floor(np.log2(tgt))
        ulp = 2.0 ** (e - 7)
        s[c] = np.float32(abs(wv[c]) / ((np.floor(tgt / ulp) + 0.5) * ulp))
    gain = rng.uniform(0.5, 2.0, 256).astype(np.float32)
    wd, sd, gd = dev_bf16(w), dev(s), dev(gain.copy())
    out = qr.uaq_fold(wd, sd, gd)
    ro, rg = oracle.uaq_fold(w, s, gain)
    assert_bitexact(host(out), ro, "folded weight")
    assert_bitexact(host(gd), rg, "gain")
    # in place, no gain
    qr.uaq_fold(wd, sd, None, inplace=True)
    assert_bitexact(host(wd), ro, "folded weight in place")


@pytest.mark.parametrize("n,k,transposed", [(296, 520, True), (136, 1040, False), (8, 8, True),
                                            (4096, 4096, True)])
def test_uaq_fold_quant_w_fused(n, k, transposed):
    """The fold and the 128x128 quantization in one pass against the oracle's fold followed
    by its block quantizer, bit for bit (folded weight, gain, codes, scales and the transposed
    copy), on ragged tile grids and the 8B step's 4096x4096 weight; rare routes included
    (signed zeros, bf16 subnormals, scales outside [2^-120, 2^121), quotients far from 1).
    Then in place, and against the two separate entry points on the GPU."""
    say("fold+quant_w", n, k, transposed)
    rng = np.random.default_rng(n + 3 * k)
    w = qr_synth.normal_bf16(81 + n, (n, k), 0.02)
    s = rng.uniform(1.5, 4.0, k).astype(np.float32)
    flat = w.reshape(-1)
    pick = rng.choice(flat.size, size=max(1, flat.size // 50), replace=False)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8040, 0x007F, 0x0080, 0x3F80], np.uint16)
    flat[pick] = specials[rng.integers(0, specials.size, pick.size)]
    s[:8] = np.array([2.0 ** -121, 1e-30, 2.0 ** 121, 1e30, 2.0 ** 127, np.float32(3.4e38),
                      1.0, 2.0 ** -60], np.float32)
    gain = rng.uniform(0.5, 2.0, k).astype(np.float32)
    ro, rg = oracle.uaq_fold(w, s, gain)
    rq, rs = oracle.quant_blocks(ro)
    wd, sd, gd = dev_bf16(w), dev(s), dev(gain.copy())
    out, q, sq, qT, sqT = qr.uaq_fold_quant_w(wd, sd, gd, transposed=transposed)
    assert_bitexact(host(out), ro, "folded weight")
    assert_bitexact(host(gd), rg, "gain")
    assert_bitexact(host(q), rq, "codes")
    assert_bitexact(host(sq), rs, "block scales")
    if transposed:
        assert_bitexact(host(qT), np.ascontiguousarray(rq.T), "transposed codes")
        assert_bitexact(host(sqT), np.ascontiguousarray(rs.T), "transposed scales")
    # the separate entry points give the same bits
    f2 = qr.uaq_fold(wd, sd)
    q2, s2, qT2, sT2 = g_quant_w(qr, f2, transposed=transposed)
    assert torch.equal(f2, out) and torch.equal(q2, q) and torch.equal(s2, sq)
    if transposed:
        assert torch.equal(qT2, qT) and torch.equal(sT2, sqT)
    # in place, no gain
    out3, q3, sq3, _, _ = qr.uaq_fold_quant_w(wd, sd, None, transposed=False, inplace=True)
    assert out3.data_ptr() == wd.data_ptr()
    assert_bitexact(host(wd), ro, "folded weight in place")
    assert torch.equal(q3, q) and torch.equal(sq3, sq)


def test_uaq_fold_quant_w_fused_strided():
    """A weight that is a column slice of a wider buffer (ld_w = 448 > k = 384): out of place
    (W' dense) and in place (W' keeps ld_w; the columns past k stay untouched)."""
    say("fold+quant_w strided")
    n, k, ld = 256, 384, 448
    rng = np.random.default_rng(17)
    full = qr_synth.normal_bf16(91, (n, ld), 0.02)
    w = np.ascontiguousarray(full[:, :k])
    s = rng.uniform(1.5, 4.0, k).astype(np.float32)
    ro, _ = oracle.uaq_fold(w, s)
    rq, rs = oracle.quant_blocks(ro)
    fd = dev_bf16(full)
    out, q, sq, qT, sqT = qr.uaq_fold_quant_w(fd[:, :k], dev(s), None, transposed=True)
    assert_bitexact(host(out), ro, "folded weight")
    assert_bitexact(host(q), rq, "codes")
    assert_bitexact(host(sq), rs, "block scales")
    assert_bitexact(host(qT), np.ascontiguousarray(rq.T), "transposed codes")
    out2, q2, sq2, _, _ = qr.uaq_fold_quant_w(fd[:, :k], dev(s), None, inplace=True)
    h = host(fd)
    assert_bitexact(np.ascontiguousarray(h[:, :k]), ro, "folded weight in place")
    assert_bitexact(np.ascontiguousarray(h[:, k:]), np.ascontiguousarray(full[:, k:]), "tail")
    assert torch.equal(q2, q) and torch.equal(sq2, sq)


@pytest.mark.parametrize("n,k", [(37, 520), (301, 1040), (1, 8)])
def test_uaq_fold_edges_and_ragged(n, k):
    """Ragged grids (rows not a multiple of 4, columns not a multiple of 512, several trips of
    the row loop) and the rare per-element routes: signed zeros, bf16 subnormals, quotients
    that overflow bf16 or fall to its subnormals, scales outside [2^-120, 2^121)."""
    say("uaq fold edges", n, k)
    rng = np.random.default_rng(n * 7 + k)
    w = qr_synth.normal_bf16(71 + n, (n, k), 0.02)
    s = rng.uniform(1.5, 4.0, k).astype(np.float32)
    flat = w.reshape(-1)
    pick = rng.choice(flat.size, size=max(1, flat.size // 20), replace=False)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8040, 0x007F, 0x7F7F, 0xFF7F, 0x0080,
                         0x3F80], np.uint16)
    flat[pick] = specials[rng.integers(0, specials.size, pick.size)]
    if k >= 8:
        s[:8] = np.array([2.0 ** -126, 2.0 ** -121, 1e-30, 2.0 ** 121, 1e30, 2.0 ** 127,
                          np.float32(3.4e38), 1.0], np.float32)
    gain = rng.uniform(0.5, 2.0, k).astype(np.float32)
    gd = dev(gain.copy())
    out = qr.uaq_fold(dev_bf16(w), dev(s), gd)
    ro, rg = oracle.uaq_fold(w, s, gain)
    assert_bitexact(host(out), ro, "folded weight")
    assert_bitexact(host(gd), rg, "gain")


# ================================================================= GEMMs

def _fprop_case(lin, x, w, out_dtype, sample=None, name="", literal=False):
    say("fprop", lin.M if lin else x.shape, name)
    xd = dev_bf16(x)
    qa, sa, _, _ = g_quant_act(qr, xd, row=True)
    ra, rsa = oracle.quant_rows(x)
    rw, rsw = oracle.quant_blocks(w)
    if w.shape[0] % 8 == 0:
        qw, sw, _, _ = g_quant_w(qr, dev_bf16(w))
        assert_bitexact(host(qw), rw, "W codes")
    else:
        # the weight quantizer takes n % 8 == 0; the GEMM takes any N, so such a weight's
        # codes come from the oracle's quantizer
        qw, sw = dev(rw), dev(rsw)
    y = g_gemm_fprop(qr, qa, sa, qw, sw, out_dtype=out_dtype)
    assert_bitexact(host(qa), ra, "A codes")
    yg = out_f64(y)
    bf = out_dtype == qr.QR_OUT_BF16
    if sample is None:
        Y, S = oracle.fprop(ra, rsa, rw, rsw)
        return assert_gemm_close(yg, Y, S, name, bf, literal)
    mi, ni = sample
    Y, S = oracle.fprop(ra, rsa, rw, rsw, sample=(mi, ni))
    return assert_gemm_close(yg[mi, ni], Y, S, name, bf, literal)


def test_fprop_tiny_fp32_full():
    lin = qr_synth.tiny_fprop()
    print(_fprop_case(lin, lin.x(), lin.w(), qr.QR_OUT_F32, name="tiny_fprop", literal=True))


# Products of these sizes with M > 64 mostly take the 64-row decode tiles (their K walks on
# 256-row tiles would be short); the comments name what a shape exercises.
@pytest.mark.parametrize("M,N,K", [(77, 200, 384), (1, 128, 128), (300, 264, 256),
                                   (129, 1000, 640), (64, 512, 1024), (256, 384, 2048),
                                   (520, 136, 384),
                                   # one K step, and ragged M and N over several row bands
                                   (300, 264, 128), (600, 520, 1152),
                                   # unsplit 256-row tiles with ragged M and N % 8 == 0: the bf16
                                   # output staged through LDS on 256x256 and on 256x128 tiles
                                   (2050, 4104, 128), (200, 16392, 512),
                                   # decode batches (M <= 64): ragged N, group counts that
                                   # are not a multiple of the four-stage ring
                                   (5, 200, 1152), (17, 1000, 384), (33, 72, 640),
                                   (64, 264, 1280), (16, 8, 128),
                                   # decode batches on weights wide enough for 128-wide tiles
                                   # (more than 256 tiles of 64 rows), ragged N
                                   (9, 16448, 256), (33, 16449, 384),
                                   # decode batches on narrow weights: K split across
                                   # workgroups (2 and 3 splits, the last one shorter)
                                   (40, 1000, 2304), (64, 520, 3200),
                                   # N % 4 != 0: the scalar tail of every output store (256x256
                                   # tiles with and without a K split, the decode kernel with
                                   # and without one, the split reduction over an odd M * N)
                                   (77, 77, 384), (2048, 4097, 128), (300, 201, 256),
                                   (5, 13, 1152), (40, 14337, 256), (64, 1001, 2304),
                                   (1, 3, 128),
                                   # the planner's row boundaries: 65 rows (the decode tiles
                                   # over two row bands, 2 K splits) and 257 rows (64x128 tiles
                                   # over five row bands)
                                   (65, 1000, 2304), (257, 7168, 1280)])
@pytest.mark.parametrize("out", [qr.QR_OUT_F32, qr.QR_OUT_BF16])
def test_fprop_shapes_full(M, N, K, out):
    x = qr_synth.normal_bf16(M + N + K, (M, K), 1.0, 7, max(1, K // 100))
    w = qr_synth.normal_bf16(M * N + K, (N, K), 0.02)
    print(_fprop_case(None, x, w, out, name=f"{M}x{N}x{K}"))


# The K-walk paths of the 256-row tiles, every output: one row band without a K split (each
# workgroup's K start rotated, the early B loads) with 1, 2, 5 and 11 K groups, where a rotation
# wraps inside a 4-group scale chunk unless it is kept on a chunk boundary (11 groups: rotations
# of 0, 7 and 3; 5 groups: 0 and 1), on 256x256 tiles (65 and 200 rows, more than 128 tiles) and
# 256x128 tiles (256 rows, 2 groups).
SINGLE_BAND = [(200, 9000, 128), (256, 9000, 256), (100, 33024, 640), (65, 33000, 1408)]


@pytest.mark.parametrize("M,N,K", SINGLE_BAND)
def test_fprop_single_band_k_walk(M, N, K):
    x = qr_synth.normal_bf16(M * 5 + N + K, (M, K), 1.0, 3, max(1, K // 100))
    w = qr_synth.normal_bf16(M + 3 * N + K, (N, K), 0.02)
    print(_fprop_case(None, x, w, qr.QR_OUT_BF16, name=f"single band {M}x{N}x{K}"))


@pytest.mark.parametrize("M,N,K", SINGLE_BAND)
def test_gemm_int8_single_band_k_walk(M, N, K):
    say("gemm_int8 single band", M, N, K)
    qa, sa, qb, sb = _int8_case(M, N, K, 5 * M + N)
    y = qr.gemm_int8(dev(qa), dev(sa), dev(qb), dev(sb), out_dtype=qr.QR_OUT_F32)
    assert np.array_equal(host(y), _int8_scaled_exact(qa, sa, qb, sb))


def test_fprop_multi_band_split_sampled():
    """256x256 tiles over five row bands with K split 3 ways (11 groups per split, the last one
    shorter; ragged M and N): the split path of the multi-band tiles, sampled outputs with every
    tile edge."""
    M, N, K = 1030, 4100, 4096
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, M, N, K) == 3 * M * N * 4
    x = qr_synth.normal_bf16(23, (M, K), 1.0, 5, 40)
    w = qr_synth.normal_bf16(29, (N, K), 0.02)
    print(_fprop_case(None, x, w, qr.QR_OUT_BF16, sample=sample_positions(M, N, 4096, seed=M + N),
                      name="multi band split 1030x4100x4096"))


def test_fprop_multi_band_xcd_rotation_sampled():
    """Tiles over five row bands without a K split (130 tiles): each XCD starts its K walk at its
    own scale chunk, 11 groups, so the start wraps inside the range; sampled outputs with every
    tile edge."""
    M, N, K = 1280, 6656, 1408
    x = qr_synth.normal_bf16(17, (M, K), 1.0, 5, 14)
    w = qr_synth.normal_bf16(19, (N, K), 0.02)
    print(_fprop_case(None, x, w, qr.QR_OUT_BF16, sample=sample_positions(M, N, 4096, seed=M + K),
                      name="multi band 1280x6656x1408"))


def test_fprop_decode_8b_full():
    lin = qr_synth.decode_8b()
    print(_fprop_case(lin, lin.x(), lin.w(), qr.QR_OUT_BF16, None, "decode_8b", literal=True))


def test_fprop_decode_8b_gate_up_full():
    """Decode batch 64 against the 8B gate+up projection (28672 rows: the 128-wide decode
    tiles); every output."""
    M, N, K = 64, 28672, 4096
    x = qr_synth.normal_bf16(M + 3 * K, (M, K), 1.0, 11, max(1, K // 100))
    w = qr_synth.normal_bf16(N + 3 * K, (N, K), 0.02)
    print(_fprop_case(None, x, w, qr.QR_OUT_BF16, None, f"{M}x{N}x{K}", literal=True))


@pytest.mark.parametrize("M,N,K", [(64, 4096, 14336), (64, 5120, 27648)])
def test_fprop_decode_narrow_full(M, N, K):
    """Decode batch 64 against the 8B down projection and the 32B one: the weight is narrow,
    so K is split across workgroups; every output."""
    x = qr_synth.normal_bf16(M + K, (M, K), 1.0, 11, max(1, K // 100))
    w = qr_synth.normal_bf16(N + K, (N, K), 0.02)
    print(_fprop_case(None, x, w, qr.QR_OUT_BF16, None, f"{M}x{N}x{K}", literal=True))


def test_fprop_prefill_8b_full():
    lin = qr_synth.prefill_8b()
    print(_fprop_case(lin, lin.x(), lin.w(), qr.QR_OUT_BF16, None, "prefill_8b", literal=True))


def _pow2_scaled(bits, exps, axis):
    """bf16 tensor with slice i along `axis` (rows or columns) multiplied by 2^exps[i % len]
    (exact in bf16 while the result stays normal)."""
    f = qr_synth.bf16_bits_to_f32(bits).astype(np.float64)
    e = np.array([exps[i % len(exps)] for i in range(f.shape[axis])], np.float64)
    f = f * (2.0 ** (e[:, None] if axis == 0 else e[None, :]))
    return qr_synth.f32_to_bf16_bits(f.astype(np.float32))


def test_fprop_extreme_group_scales():
    """Group scales far from 1 inside the documented domain (every product sA * sB of two
    non-zero group scales at least 2^-126, every output below 2^128), zero groups (scale 0)
    and groups of negative zeros (codes 0x80): rows of A carry 2^-54 .. 2^60, 128-row blocks
    of the weight 2^-50 .. 2^56, so the scale products span about 2^-123 .. 2^101."""
    say("fprop extreme scales")
    M, N, K = 300, 384, 768
    x = _pow2_scaled(qr_synth.normal_bf16(61, (M, K), 1.0, 62, 8), [-54, -30, 0, 30, 60], 0)
    x[3::7, 256:384] = 0x0000                          # a zero group per 7th row
    x[5::7, 512:640] = 0x8000                          # a group of negative zeros
    w = _pow2_scaled(qr_synth.normal_bf16(63, (N, K), 0.02), [-50] * 128 + [0] * 128 + [56] * 128, 0)
    w[128:256, 384:512] = 0x0000                       # a zero weight block
    for out in (qr.QR_OUT_F32, qr.QR_OUT_BF16):
        print(_fprop_case(None, x, w, out, None, f"extreme scales out={out}"))
    # the tile path with a K split over the same operands (M <= 256: 2 tiles of 256x256)
    print(_fprop_case(None, np.ascontiguousarray(x[:200]), w, qr.QR_OUT_F32, None,
                      "extreme scales, K split"))


def test_wgrad_extreme_group_scales():
    """WGrad's outer-product promotion with per-channel scales 2^-50 .. 2^56 on both operands,
    a zero token group and a group of negative zeros, compared in full."""
    say("wgrad extreme scales")
    M, N, K = 384, 264, 520
    dy = _pow2_scaled(qr_synth.normal_bf16(65, (M, N), 1e-3), [-40, -10, 0, 20, 50], 1)
    x = _pow2_scaled(qr_synth.normal_bf16(66, (M, K), 1.0, 67, 5), [-50, 0, 30, 56], 1)
    dy[128:256, 7::11] = 0x0000
    x[256:384, 3::13] = 0x8000
    _, _, qdyT, sdyT = g_quant_act(qr, dev_bf16(dy), row=False, col=True)
    _, _, qxT, sxT = g_quant_act(qr, dev_bf16(x), row=False, col=True)
    rdyT, rsdyT = oracle.quant_cols_T(dy)
    rxT, rsxT = oracle.quant_cols_T(x)
    assert_bitexact(host(qdyT), rdyT, "dY^T codes")
    assert_bitexact(host(qxT), rxT, "X^T codes")
    Y, S = oracle.wgrad(rdyT, rsdyT, rxT, rsxT)
    for out in (qr.QR_OUT_F32, qr.QR_OUT_BF16):
        dw = g_gemm_wgrad(qr, qdyT, sdyT, qxT, sxT, out_dtype=out)
        print("wgrad extreme", assert_gemm_close(out_f64(dw), Y, S, "wgrad", out == qr.QR_OUT_BF16))


def test_fprop_empty_and_zero_k():
    say("fprop empty / K=0")
    a = torch.zeros((4, 0), dtype=torch.uint8, device="cuda")
    y = torch.full((4, 8), 7.0, device="cuda")
    qr.qr_gemm_fp8_bsfprop(a, torch.zeros(4, device="cuda"), a, torch.zeros(1, device="cuda"),
                           4, 8, 0, y, qr.QR_OUT_F32)
    assert float(y.abs().max()) == 0.0
    qr.qr_gemm_fp8_bsfprop(None, None, None, None, 0, 8, 128, y, qr.QR_OUT_F32)   # M = 0
    torch.cuda.synchronize()


def _backward_operands():
    lin = qr_synth.prefill_8b()
    x, w, dy = lin.x(), lin.w(), qr_synth.backward_8b_dy()
    return x, w, dy


def test_backward_8b_dgrad_wgrad_full():
    say("backward_8b")
    x, w, dy = _backward_operands()
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    qdy, sdy, qdyT, sdyT = g_quant_act(qr, dyd, row=True, col=True)
    _, _, qxT, sxT = g_quant_act(qr, xd, row=False, col=True)
    _, _, qwT, swT = g_quant_w(qr, wd, transposed=True)
    dx = g_gemm_dgrad(qr, qdy, sdy, qwT, swT)
    dw = g_gemm_wgrad(qr, qdyT, sdyT, qxT, sxT)
    rdy, rsdy = oracle.quant_rows(dy)
    rdyT, rsdyT = oracle.quant_cols_T(dy)
    rxT, rsxT = oracle.quant_cols_T(x)
    rw, rsw = oracle.quant_blocks(w)
    assert_bitexact(host(qwT), np.ascontiguousarray(rw.T), "W^T codes")
    assert_bitexact(host(qxT), rxT, "X^T codes")
    assert_bitexact(host(qdy), rdy, "dY row codes")
    assert_bitexact(host(qdyT), rdyT, "dY^T codes")
    Y, S = oracle.dgrad(rdy, rsdy, rw, rsw)
    print("dgrad", assert_gemm_close(out_f64(dx), Y, S, "dgrad", True, literal=True))
    del Y, S
    Y, S = oracle.wgrad(rdyT, rsdyT, rxT, rsxT)
    print("wgrad", assert_gemm_close(out_f64(dw), Y, S, "wgrad", True, literal=True))


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (384, 200, 384), (128, 77, 1024),
                                   (1024, 136, 512),
                                   # WGrad on 256x256 tiles (N > 256): ragged rows, and a
                                   # contraction of one group (M = 128 tokens)
                                   (256, 520, 384), (128, 300, 256)])
def test_dgrad_wgrad_small_full(M, N, K):
    """Full comparison on small backward shapes: M tokens, N output features, K inputs."""
    say("dgrad/wgrad small", M, N, K)
    x = qr_synth.normal_bf16(M + K, (M, K), 1.0, 3, 2)
    dy = qr_synth.normal_bf16(M + N + 1, (M, N), 1e-3)
    n_pad = ((N + 127) // 128) * 128 if N % 128 else N
    # DGrad contracts over N: pad N to whole groups with zero gradient columns and weights
    dy_p = np.zeros((M, n_pad), np.uint16)
    dy_p[:, :N] = dy
    w = np.zeros((n_pad, K), np.uint16)
    w[:N] = qr_synth.normal_bf16(N * K, (N, K), 0.02)
    qdy, sdy, qdyT, sdyT = g_quant_act(qr, dev_bf16(dy_p), row=True, col=True)
    _, _, qxT, sxT = g_quant_act(qr, dev_bf16(x), row=False, col=True)
    _, _, qwT, swT = g_quant_w(qr, dev_bf16(w), transposed=True)
    for out in (qr.QR_OUT_F32, qr.QR_OUT_BF16):
        dx = g_gemm_dgrad(qr, qdy, sdy, qwT, swT, out_dtype=out)
        rdy, rsdy = oracle.quant_rows(dy_p)
        rw, rsw = oracle.quant_blocks(w)
        Y, S = oracle.dgrad(rdy, rsdy, rw, rsw)
        assert_gemm_close(out_f64(dx), Y, S, "dgrad", out == qr.QR_OUT_BF16)
        dw = g_gemm_wgrad(qr, qdyT, sdyT, qxT, sxT, out_dtype=out)
        rdyT, rsdyT = oracle.quant_cols_T(dy_p)
        rxT, rsxT = oracle.quant_cols_T(x)
        Y, S = oracle.wgrad(rdyT, rsdyT, rxT, rsxT)
        assert_gemm_close(out_f64(dw), Y, S, "wgrad", out == qr.QR_OUT_BF16)


@pytest.mark.parametrize("M,N,K", [(48, 384, 520), (8, 128, 1000), (48, 2304, 384)])
def test_dgrad_decode_batch_full(M, N, K):
    """DGrad with a small token count takes the 64-row decode tiles; full comparison."""
    say("dgrad small M", M, N, K)
    dy = qr_synth.normal_bf16(M + N + 5, (M, N), 1e-3)
    w = qr_synth.normal_bf16(N * K + 5, (N, K), 0.02)
    qdy, sdy, _, _ = g_quant_act(qr, dev_bf16(dy), row=True)
    _, _, qwT, swT = g_quant_w(qr, dev_bf16(w), transposed=True)
    rdy, rsdy = oracle.quant_rows(dy)
    rw, rsw = oracle.quant_blocks(w)
    for out in (qr.QR_OUT_F32, qr.QR_OUT_BF16):
        dx = g_gemm_dgrad(qr, qdy, sdy, qwT, swT, out_dtype=out)
        Y, S = oracle.dgrad(rdy, rsdy, rw, rsw)
        assert_gemm_close(out_f64(dx), Y, S, "dgrad", out == qr.QR_OUT_BF16)


@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_decode_32b_set_full(idx):
    lin = qr_synth.decode_32b_set()[idx]
    say("decode_32b", lin.name, lin.M, lin.N, lin.K)
    w, s, x = lin.w(), lin.uaq_s(), lin.x()
    wd = dev_bf16(w)
    wf = qr.uaq_fold(wd, dev(s))
    rwf, _ = oracle.uaq_fold(w, s)
    assert_bitexact(host(wf), rwf, "folded W")
    del wd
    print(_fprop_case(lin, x, rwf, qr.QR_OUT_BF16, None, lin.name, literal=True))


@pytest.mark.parametrize("M,N,K", [(64, 14336, 4096),    # decode, no split
                                   (64, 4096, 14336),    # decode, K split across workgroups
                                   (256, 7168, 5120),    # 256x256 tiles, 8 K splits
                                   (200, 640, 1024)])    # ragged M, 3 tiles x 8 K splits
def test_gemm_deterministic(M, N, K):
    """Repeated calls give bit-identical outputs, also where K is split (the partial sums
    are added in split order, never in arrival order)."""
    say("determinism", M, N, K)
    x = qr_synth.normal_bf16(M + 2 * K, (M, K), 1.0, 13, max(1, K // 100))
    w = qr_synth.normal_bf16(N + 3 * K, (N, K), 0.02)
    qa, sa, _, _ = g_quant_act(qr, dev_bf16(x), row=True)
    qw, sw, _, _ = g_quant_w(qr, dev_bf16(w))
    for out in (qr.QR_OUT_F32, qr.QR_OUT_BF16):
        ys = [host(g_gemm_fprop(qr, qa, sa, qw, sw, out_dtype=out)) for _ in range(3)]
        assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2]), (M, N, K, out)
