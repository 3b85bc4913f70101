"""Seeded random shapes through every GEMM, quantizer and norm plan, each compared in full with the
oracle: the shapes are drawn across the planner's regions (decode batches of at most 64 rows,
65..256-row batches, larger products), with ragged sizes and contraction lengths of 1 to 20
groups, so that tile choices, K splits (and their three-groups rule) and ragged tails are met
in combinations the hand-picked cases do not list.  The draw is fixed by the seed.

QR_RANDOM_SHAPES_SEED (default 20261203) and QR_RANDOM_SHAPES_SCALE (default 1, a multiplier
on every case count) widen the sweep: each family draws from the seed plus its own offset."""
import os

import numpy as np
import pytest
import torch

import fp8_block_scaled_qr_amd as qr
import oracle
import qr_synth
from gpu_util import (assert_bitexact, assert_gemm_close, check_norm_y, check_w4a16, dev,
                      dev_bf16, g_gemm_dgrad, g_gemm_fprop, g_gemm_wgrad, g_quant_act, g_quant_w,
                      host, out_f64)

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qr.load()


_SEED = int(os.environ.get("QR_RANDOM_SHAPES_SEED", "20261203"))
_SCALE = int(os.environ.get("QR_RANDOM_SHAPES_SCALE", "1"))


def _draw(seed, count, make):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [make(rng) for _ in range(count)]


def _fprop_shape(rng):
    region = rng.integers(0, 3)
    M = int(rng.integers(1, 65) if region == 0 else rng.integers(65, 257) if region == 1
            else rng.integers(257, 700))
    N = int(rng.integers(1, 250)) * 8 if rng.random() < 0.8 else int(rng.integers(1, 2000))
    K = 128 * int(rng.integers(1, 21))
    return M, N, K


FPROP_SHAPES = _draw(_SEED + 0, 32 * _SCALE, _fprop_shape)


@pytest.mark.parametrize("M,N,K", FPROP_SHAPES)
def test_fprop_random_shape(M, N, K):
    print(f"[random fprop] {M}x{N}x{K}", flush=True)
    x = qr_synth.normal_bf16(M * 3 + N + K, (M, K), 1.0, 5, max(1, K // 100))
    w = qr_synth.normal_bf16(M + N * 7 + K, (N, K), 0.02)
    qa, sa, _, _ = g_quant_act(qr, dev_bf16(x), row=True)
    ra, rsa = oracle.quant_rows(x)
    assert_bitexact(host(qa), ra, "A codes")
    rw, rsw = oracle.quant_blocks(w)
    if N % 8 == 0:
        qw, sw, _, _ = g_quant_w(qr, dev_bf16(w))
        assert_bitexact(host(qw), rw, "W codes")
    else:
        qw, sw = dev(rw), dev(rsw)   # the weight quantizer takes n % 8 == 0
    Y, S = oracle.fprop(ra, rsa, rw, rsw)
    out = qr.QR_OUT_BF16 if (M + N + K) % 2 else qr.QR_OUT_F32
    y = g_gemm_fprop(qr, qa, sa, qw, sw, out_dtype=out)
    assert_gemm_close(out_f64(y), Y, S, f"fprop {M}x{N}x{K}", out == qr.QR_OUT_BF16)


def _backward_shape(rng):
    M = 128 * int(rng.integers(1, 7))    # tokens: WGrad's contraction
    N = 128 * int(rng.integers(1, 13))   # output features: DGrad's contraction
    K = 8 * int(rng.integers(1, 200))    # input features
    return M, N, K


BACKWARD_SHAPES = _draw(_SEED + 1, 12 * _SCALE, _backward_shape)


@pytest.mark.parametrize("M,N,K", BACKWARD_SHAPES)
def test_dgrad_wgrad_random_shape(M, N, K):
    print(f"[random dgrad/wgrad] {M}x{N}x{K}", flush=True)
    x = qr_synth.normal_bf16(M + 2 * K, (M, K), 1.0, 3, 2)
    dy = qr_synth.normal_bf16(M + N + 11, (M, N), 1e-3)
    w = qr_synth.normal_bf16(N * 5 + K, (N, K), 0.02)
    qdy, sdy, qdyT, sdyT = g_quant_act(qr, dev_bf16(dy), row=True, col=True)
    _, _, qxT, sxT = g_quant_act(qr, dev_bf16(x), row=False, col=True)
    _, _, qwT, swT = g_quant_w(qr, dev_bf16(w), transposed=True)
    out = qr.QR_OUT_BF16 if (M + N + K) % 3 else qr.QR_OUT_F32
    rdy, rsdy = oracle.quant_rows(dy)
    rw, rsw = oracle.quant_blocks(w)
    Y, S = oracle.dgrad(rdy, rsdy, rw, rsw)
    dx = g_gemm_dgrad(qr, qdy, sdy, qwT, swT, out_dtype=out)
    assert_gemm_close(out_f64(dx), Y, S, f"dgrad {M}x{N}x{K}", out == qr.QR_OUT_BF16)
    rdyT, rsdyT = oracle.quant_cols_T(dy)
    rxT, rsxT = oracle.quant_cols_T(x)
    assert_bitexact(host(qdyT), rdyT, "dY column codes")
    assert_bitexact(host(qxT), rxT, "X column codes")
    Y, S = oracle.wgrad(rdyT, rsdyT, rxT, rsxT)
    dw = g_gemm_wgrad(qr, qdyT, sdyT, qxT, sxT, out_dtype=out)
    assert_gemm_close(out_f64(dw), Y, S, f"wgrad {M}x{N}x{K}", out == qr.QR_OUT_BF16)


def _int8_shape(rng):
    M = int(rng.integers(1, 65) if rng.random() < 0.4 else rng.integers(65, 600))
    N = int(rng.integers(1, 1600))
    K = 128 * int(rng.integers(1, 21))
    return M, N, K


INT8_SHAPES = _draw(_SEED + 2, 12 * _SCALE, _int8_shape)


@pytest.mark.parametrize("M,N,K", INT8_SHAPES)
def test_int8_random_shape(M, N, K):
    """The INT8 product is exact in int32 and scaled once, so the GPU output equals the
    oracle's scaled exact sum bit for bit (fp32 out)."""
    print(f"[random int8] {M}x{N}x{K}", flush=True)
    x = qr_synth.normal_bf16(M + 13 * K, (M, K), 1.0, 7, max(1, K // 100))
    w = qr_synth.normal_bf16(N + 17 * K, (N, K), 0.02)
    qa, sa = qr.quant_int8(dev_bf16(x))
    qw, sw = qr.quant_int8(dev_bf16(w))
    ra, rsa = oracle.quant_int8_rows(x)
    rw, rsw = oracle.quant_int8_rows(w)
    assert_bitexact(host(qa), ra, "activation codes")
    assert_bitexact(host(sa), rsa, "activation scales")
    assert_bitexact(host(qw), rw, "weight codes")
    assert_bitexact(host(sw), rsw, "weight scales")
    y = qr.gemm_int8(qa, sa, qw, sw, out_dtype=qr.QR_OUT_F32)
    ref = oracle.gemm_int8(ra, rsa, rw, rsw)
    exact = (ra.astype(np.int64) @ rw.astype(np.int64).T).astype(np.float32)
    want = exact * (rsa.astype(np.float32)[:, None] * rsw.astype(np.float32)[None, :])
    assert np.array_equal(host(y), want), "fp32 output of the scaled exact sum"
    err = np.abs(out_f64(y) - ref)
    assert np.all(err <= 2.0 ** -22 * np.abs(ref)), "three binary32 roundings of the fp64 oracle"


def _quant_shape(rng):
    return 8 * int(rng.integers(1, 90)), 8 * int(rng.integers(1, 160))


QUANT_SHAPES = _draw(_SEED + 3, 12 * _SCALE, _quant_shape)


@pytest.mark.parametrize("rows,cols", QUANT_SHAPES)
def test_quant_dual_random_shape(rows, cols):
    print(f"[random quant] {rows}x{cols}", flush=True)
    x = qr_synth.normal_bf16(rows * 3 + cols, (rows, cols), 1.0, 9, max(1, cols // 100))
    q, s, qT, sT = g_quant_act(qr, dev_bf16(x), row=True, col=True)
    rq, rs = oracle.quant_rows(x)
    rqT, rsT = oracle.quant_cols_T(x)
    assert_bitexact(host(q), rq, "row codes")
    assert_bitexact(host(s), rs, "row scales")
    assert_bitexact(host(qT), rqT, "column codes")
    assert_bitexact(host(sT), rsT, "column scales")
    w = qr_synth.normal_bf16(rows + cols * 5, (rows, cols), 0.02)
    qw, sw, qwT, swT = g_quant_w(qr, dev_bf16(w), transposed=True)
    rw, rsw = oracle.quant_blocks(w)
    assert_bitexact(host(qw), rw, "block codes")
    assert_bitexact(host(sw), rsw, "block scales")
    assert_bitexact(host(qwT), np.ascontiguousarray(rw.T), "transposed block codes")
    assert_bitexact(host(swT), np.ascontiguousarray(rsw.T), "transposed block scales")


def _norm_shape(rng):
    rows = 8 * int(rng.integers(1, 80))
    cols = 8 * int(rng.integers(1, 1000) if rng.random() < 0.7 else rng.integers(1000, 4000))
    return rows, cols


NORM_SHAPES = _draw(_SEED + 4, 12 * _SCALE, _norm_shape)


@pytest.mark.parametrize("rows,cols", NORM_SHAPES)
def test_rmsnorm_random_shape(rows, cols):
    """Both norm entry points: y as the oracle's RMSNorm (one bf16 ulp allowed only next to a
    midpoint), and every code and scale bit-exact against the oracle's quantizers of the
    GPU's y; the dual entry point's y equals the single-layout one's for the same input."""
    print(f"[random rmsnorm] {rows}x{cols}", flush=True)
    rng = np.random.Generator(np.random.PCG64(rows * 31 + cols))
    h = qr_synth.normal_bf16(rows * 7 + cols, (rows, cols), 1.0, 4, max(1, cols // 100))
    g = rng.uniform(0.5, 6.0, cols).astype(np.float32)
    eps = 1e-6 if rows % 16 else 1e-5
    hd, gd = dev_bf16(h), dev(g)
    y, q, s = qr.rmsnorm_quant(hd, gd, eps)
    yg = host(y)
    check_norm_y(yg, h, g, eps)
    rq, rs = oracle.quant_rows(np.ascontiguousarray(yg))
    assert_bitexact(host(q), rq, "row codes of y")
    assert_bitexact(host(s), rs, "row scales of y")
    inv, y2, q2, s2, qT2, sT2 = qr.rmsnorm_quant_dual(hd, gd, eps, want_y=True)
    yg2 = host(y2)
    check_norm_y(yg2, h, g, eps)
    rqT, rsT = oracle.quant_cols_T(np.ascontiguousarray(yg2))
    rq2, rs2 = oracle.quant_rows(np.ascontiguousarray(yg2))
    assert_bitexact(host(q2), rq2, "dual row codes of y")
    assert_bitexact(host(s2), rs2, "dual row scales of y")
    assert_bitexact(host(qT2), rqT, "dual column codes of y")
    assert_bitexact(host(sT2), rsT, "dual column scales of y")


def _w4_shape(rng):
    M = int(rng.integers(1, 65) if rng.random() < 0.6 else rng.integers(65, 300))
    N = int(rng.integers(1, 1500))
    K = 128 * int(rng.integers(1, 48))
    return M, N, K


W4_SHAPES = _draw(_SEED + 5, 12 * _SCALE, _w4_shape)


@pytest.mark.parametrize("M,N,K", W4_SHAPES)
def test_w4a16_random_shape(M, N, K):
    """4-bit weight codes and scales bit-exact; the product within K 2^-23 sum |x w| t of the
    oracle (plus the bf16 rounding for bf16 output)."""
    print(f"[random w4a16] {M}x{N}x{K}", flush=True)
    x = qr_synth.normal_bf16(M * 5 + K, (M, K), 1.0, 6, max(1, K // 100))
    w = qr_synth.normal_bf16(N * 3 + K + 1, (N, K), 0.02)
    codes, bs, t = qr.quant_nvfp4(dev_bf16(w))
    hc, hb = host(codes), host(bs)
    rc, rb, rt = oracle.quant_nvfp4(w)
    assert_bitexact(hc, rc, "4-bit codes")
    assert_bitexact(hb, rb, "block scales")
    assert_bitexact(host(t), np.array([rt], np.float32), "tensor scale")
    out = qr.QR_OUT_BF16 if (M + N) % 2 else qr.QR_OUT_F32
    y = out_f64(qr.gemm_w4a16(dev_bf16(x), codes, bs, t, out_dtype=out))
    Y = oracle.gemm_w4a16(x, hc, hb, rt)
    absw = oracle.gemm_w4a16(x & np.uint16(0x7FFF), hc & np.uint8(0x77), hb, rt)   # sum |x w| t
    check_w4a16(y, Y, K * 2.0 ** -23 * np.abs(absw))
