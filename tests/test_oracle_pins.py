"""Pins of the reference oracle against what the pages and mathematics fix (CPU only).

Each test checks the oracle against something other than itself: hand-derived values from
the format definition, torch's float8_e4m3fn codec (a library routine), brute-force nearest
search, exact rational arithmetic (fractions), integer matmul special cases, closed forms and
invariants.  A plausible mistake anywhere in the oracle (wrong rounding direction, dropped
saturation, sign of zero, transposed scale index, wrong group boundary, a sign or index error
in the GEMM) fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import qr_synth
from exact_ref import (bf16_bits_of, e4m3_nearest, e4m3_values_torch, f32_of, rn32, rn_bf16)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def bf16_f32(bits):
    return qr_synth.bf16_bits_to_f32(np.asarray(bits, np.uint16))


# ============================================================== E4M3 codec

def test_anchor_codes_hand_derived():
    n = 0
    for parts in _golden_lines("e4m3_anchor_codes.txt"):
        v = np.float32(parts[0])
        assert Fraction(float(v)) == Fraction(parts[0].lstrip("-")) * (-1 if parts[0].startswith("-") else 1) \
            or parts[0] in ("-0.0",)
        assert oracle.e4m3_encode(v) == int(parts[1], 16), parts
        n += 1
    assert n >= 25


def test_decode_matches_torch_float8_all_codes():
    mine = oracle.e4m3_decode_table()
    ref = e4m3_values_torch()
    nan = np.isnan(ref)
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert math.copysign(1.0, mine[0x80]) == -1.0      # 0x80 is -0


def test_decode_structure():
    v = oracle.e4m3_decode_table()
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # monotone over 0x00..0x7E
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6 and pos[0x38] == 1.0
    assert np.array_equal(v[0x80:0xFF], -pos)           # sign symmetry
    finite = v[~np.isnan(v)]
    assert len(set(finite.tolist())) == 253             # +0 and -0 compare equal


def test_roundtrip_all_finite_codes():
    v = oracle.e4m3_decode_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(np.float32(v[c]) if c != 0x80 else np.float32(-0.0)) == c


def _midpoint_probe_values():
    pos = oracle.e4m3_decode_table()[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)          # exact in binary32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    vals = [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
            pos.astype(np.float32), np.nextafter(pos.astype(np.float32), np.float32(np.inf)),
            np.array([447.99997, 448.0, 448.00003, 463.99997, 464.0, 464.00003, 1e30,
                      np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45, 2.0 ** -10,
                      np.nextafter(np.float32(2.0 ** -10), np.float32(1))], np.float32)]
    rng = np.random.default_rng(7)
    for sc in (1e-4, 1e-2, 1.0, 30.0, 300.0):
        vals.append((rng.standard_normal(4000) * sc).astype(np.float32))
    v = np.concatenate(vals)
    return np.concatenate([v, -v])


def test_encode_matches_bruteforce_nearest():
    v = _midpoint_probe_values()
    mine = oracle.e4m3_encode_array(v)
    ref = np.array([e4m3_nearest(x) for x in v], np.uint8)
    bad = np.flatnonzero(mine != ref)
    assert bad.size == 0, [(float(v[i]), hex(mine[i]), hex(ref[i])) for i in bad[:10]]


def test_encode_matches_torch_cast_below_448():
    rng = np.random.default_rng(11)
    v = np.concatenate([(rng.standard_normal(200000) * s).astype(np.float32)
                        for s in (1e-3, 0.05, 1.0, 40.0)])
    v = v[np.abs(v) < 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode_array(v), ref)


def test_encode_saturates_every_binade_above_448():
    big = np.float32(448.0) * (np.float32(2.0) ** np.arange(0, 120, dtype=np.float32))
    big = np.concatenate([big, np.nextafter(big, np.float32(np.inf)), [np.finfo(np.float32).max]])
    big = big[np.isfinite(big)].astype(np.float32)
    assert np.all(oracle.e4m3_encode_array(big) == 0x7E)
    assert np.all(oracle.e4m3_encode_array(-big) == 0xFE)


# ============================================================== scale and quotient

def test_group_scale_exact_for_every_bf16_amax():
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint16)         # every finite non-negative bf16
    amax = bf16_f32(bits)
    # drive the real quantizer: each row's first element is the group's amax
    x = np.zeros((bits.size, 128), np.uint16)
    x[:, 0] = bits
    _, s = oracle.quant_rows(x)
    s = s[:, 0]
    # exact rational reference on a deterministic subsample + library IEEE division on all
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    for i in range(0, bits.size, 97):
        assert Fraction(float(s[i])) == rn32(Fraction(float(amax[i])) / 448), hex(bits[i])


def _groups_for_amax(amax_bits):
    """bf16 rows: a group per 127 values x with |x| <= amax, first element = amax."""
    allb = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    allv = bf16_f32(allb)
    ok = np.isfinite(allv) & (np.abs(allv) <= bf16_f32(np.uint16(amax_bits)))
    xs = allb[ok]
    pad = (-xs.size) % 127
    xs = np.concatenate([xs, np.zeros(pad, np.uint16)])
    body = xs.reshape(-1, 127)
    rows = np.empty((body.shape[0], 128), np.uint16)
    rows[:, 0] = amax_bits
    rows[:, 1:] = body
    return rows


AMAX_SAMPLES = [0x3F80, 0x43E0, 0x4000, 0x3DCD, 0x4120, 0x3C23, 0x4B00, 0x7F7F, 0x0080, 0x0001,
                0x0237, 0x1A2B, 0x2F11, 0x3A83, 0x3B12, 0x3FFF, 0x447A, 0x5F00, 0x60C1, 0x7000]


@pytest.mark.parametrize("amax_bits", AMAX_SAMPLES)
def test_codes_exhaustive_over_bf16_for_sampled_amax(amax_bits):
    """Every bf16 x with |x| <= amax: oracle code == E4M3_RNE_SAT(IEEE binary32 x/s)."""
    rows = _groups_for_amax(amax_bits)
    q, s = oracle.quant_rows(rows)
    sc = np.float32(bf16_f32(np.uint16(amax_bits)).item()) / np.float32(448.0)
    assert np.all(s[:, 0] == sc)
    x = bf16_f32(rows)
    if sc == 0:
        v = x
    else:
        with np.errstate(over="ignore"):
            v = (x / sc).astype(np.float32)                   # IEEE division (library)
    small = np.abs(v) < 448
    ref = np.where(np.signbit(v), np.uint8(0xFE), np.uint8(0x7E))
    ref[small] = torch.from_numpy(v[small]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    # exact rational check on a subsample: the quotient itself is correctly rounded
    flat_x, flat_q = x.ravel(), q.ravel()
    for i in range(0, flat_x.size, 211):
        if sc != 0:
            exact = rn32(Fraction(float(flat_x[i])) / Fraction(float(sc)))
            xv = float(exact) if exact != 0 else (-0.0 if np.signbit(flat_x[i]) else 0.0)
            assert flat_q[i] == e4m3_nearest(xv)


def test_amax_element_encodes_to_448_and_zero_group():
    x = qr_synth.normal_bf16(5, (64, 512), 1.0)
    q, s = oracle.quant_rows(x)
    xf = bf16_f32(x)
    for r in range(64):
        for g in range(4):
            seg = xf[r, g * 128:(g + 1) * 128]
            i = int(np.argmax(np.abs(seg)))
            assert q[r, g * 128 + i] == (0xFE if seg[i] < 0 else 0x7E)
    z = np.zeros((2, 128), np.uint16)
    z[1, ::2] = 0x8000                                       # negative zeros
    qz, sz = oracle.quant_rows(z)
    assert np.all(sz == 0)
    assert np.array_equal(qz[0], np.zeros(128, np.uint8))
    assert np.array_equal(qz[1, ::2], np.full(64, 0x80, np.uint8))
    assert np.array_equal(qz[1, 1::2], np.zeros(64, np.uint8))


def test_per_element_error_bound():
    """|x/s - dq(q)| <= half an E4M3 step at |dq(q)| unless saturated (where |x/s| > 448)."""
    x = qr_synth.normal_bf16(9, (256, 512), 1.0, 10, 4)
    q, s = oracle.quant_rows(x)
    v = bf16_f32(x).astype(np.float64) / np.repeat(s, 128, axis=1).astype(np.float64)
    d = oracle.e4m3_decode_table()[q]
    a = np.abs(d)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_step = np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
    # a value rounding up into the next binade sits at most half a step of the lower binade
    half_step = np.maximum(half_step, np.where(a == 2.0 ** e, 2.0 ** (e - 5), 0))
    err = np.abs(v - d)
    sat = np.abs(v) > 448
    assert np.all(err[~sat] <= half_step[~sat] * (1 + 2.0 ** -20))
    assert np.all(np.abs(d[sat]) == 448)


# ============================================================== quantizer layouts

def test_column_groups_equal_row_groups_of_transpose():
    x = qr_synth.normal_bf16(21, (384, 200), 1.0, 22, 3)
    qT, sT = oracle.quant_cols_T(x)
    q2, s2 = oracle.quant_rows(np.ascontiguousarray(x.T))
    assert np.array_equal(qT, q2) and np.array_equal(sT, s2)


def test_block_quant_of_transpose_is_transpose():
    w = qr_synth.normal_bf16(23, (384, 256), 0.02)
    q, s = oracle.quant_blocks(w)
    qt, st = oracle.quant_blocks(np.ascontiguousarray(w.T))
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def _weight_with_special_blocks():
    """Ragged bf16 weight (partial blocks in both directions) with one outlier block (x1000),
    one tiny-amax block (x2^-120: its scale is a binary32 subnormal), one all-zero block and
    one block of negative zeros and tiny negatives (their quotients round to the signed zero)."""
    w = qr_synth.normal_bf16(33, (392, 264), 0.02)
    f = bf16_f32(w)
    f[128:256, 0:128] *= np.float32(1000.0)
    f[0:128, 128:256] *= np.float32(2.0 ** -120)
    f[256:384, 128:256] = 0.0
    f[256:392, 256:264] = -0.0
    f[260, 258] = np.float32(-2.0 ** -40)          # tiny next to the block's amax below
    f[300, 260] = np.float32(3.0)
    return qr_synth.f32_to_bf16_bits(f)


def test_block_codes_against_library_division_and_torch_cast():
    """The 128x128 codes, rebuilt from library routines only: the block amax by numpy, the
    scale and the quotient by numpy's IEEE binary32 division, the code by torch's
    float8_e4m3fn cast below 448 and saturation at or above it (Jet-RL notes, fine-grained
    GEMM quantization: weights in 128x128 blocks, one scale each)."""
    w = _weight_with_special_blocks()
    q, s = oracle.quant_blocks(w)
    f = bf16_f32(w)
    n, k = f.shape
    nbi, nbj = -(-n // 128), -(-k // 128)
    s_ref = np.empty((nbi, nbj), np.float32)
    for bi in range(nbi):
        for bj in range(nbj):
            blk = f[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            s_ref[bi, bj] = np.float32(np.abs(blk).max()) / np.float32(448.0)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert s_ref[0, 1] < np.finfo(np.float32).tiny and s_ref[0, 1] > 0   # subnormal scale
    assert s_ref[2, 1] == 0 and s_ref[1, 0] > 100 * s_ref[0, 0]
    s_el = np.repeat(np.repeat(s_ref, 128, axis=0), 128, axis=1)[:n, :k]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        v = np.where(s_el == 0, f, f / s_el).astype(np.float32)
    ref = np.where(np.signbit(v), np.uint8(0xFE), np.uint8(0x7E))
    small = np.abs(v) < 448
    ref[small] = torch.from_numpy(v[small]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.argwhere(q != ref)
    assert bad.size == 0, [(tuple(i), hex(q[tuple(i)]), hex(ref[tuple(i)])) for i in bad[:8]]
    # the zero block keeps each element's sign of zero; the amax element of each block is +-448
    assert np.all(q[256:384, 128:256] == 0x00) and np.all(q[256:392, 256:264][f[256:392, 256:264] == 0] == 0x80)
    assert q[260, 258] == 0x80
    for bi in range(nbi):
        for bj in range(nbj):
            blk = f[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            if s_ref[bi, bj] > 0:
                i, j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                assert q[bi * 128 + i, bj * 128 + j] in (0x7E, 0xFE)


def test_block_codes_exact_rationals_subsample():
    """Every 37th code of the special-block weight against the exact rational quotient
    rounded once to binary32, then the nearest E4M3 value by search."""
    w = _weight_with_special_blocks()
    q, s = oracle.quant_blocks(w)
    f = bf16_f32(w)
    n, k = f.shape
    flat = np.arange(n * k)
    picks = np.concatenate([flat[::37], [128 * k + 5, 5 * k + 130, 260 * k + 258, 300 * k + 260]])
    for idx in picks:
        r, c = divmod(int(idx), k)
        x = float(f[r, c])
        amax = Fraction(float(np.abs(f[r // 128 * 128:(r // 128 + 1) * 128,
                                       c // 128 * 128:(c // 128 + 1) * 128]).max()))
        sc = rn32(amax / 448)
        assert Fraction(float(s[r // 128, c // 128])) == sc
        if sc == 0:
            xv = x
        else:
            qv = rn32(Fraction(x) / sc)
            xv = float(qv) if qv != 0 else (-0.0 if np.signbit(x) else 0.0)
        assert q[r, c] == e4m3_nearest(xv), (r, c, x, hex(q[r, c]))


def test_block_scale_is_max_of_row_group_amax():
    """A 128x128 block's amax is the max over its 128 rows' 1x128 amaxes, and s = amax/448 is
    monotone, so the block scale equals the max of the row-group scales."""
    w = qr_synth.normal_bf16(25, (256, 384), 0.02)
    _, sb = oracle.quant_blocks(w)
    _, sr = oracle.quant_rows(w)
    assert np.array_equal(sb, sr.reshape(2, 128, 3).max(axis=1))


def test_power_of_two_invariance():
    x = qr_synth.normal_bf16(27, (128, 384), 1.0, 28, 2)
    q, s = oracle.quant_rows(x)
    for j in (-20, -3, 1, 5, 30):
        x2 = qr_synth.f32_to_bf16_bits(bf16_f32(x) * np.float32(2.0 ** j))
        q2, s2 = oracle.quant_rows(x2)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))


def test_partial_group_equals_zero_padded():
    x = qr_synth.normal_bf16(29, (50, 200), 1.0)
    q, s = oracle.quant_rows(x)
    xp = np.zeros((50, 256), np.uint16)
    xp[:, :200] = x
    qp, sp = oracle.quant_rows(xp)
    assert np.array_equal(q, qp[:, :200]) and np.array_equal(s, sp)
    qT, sT = oracle.quant_cols_T(np.ascontiguousarray(x.T))      # rows = 200: partial group
    assert np.array_equal(qT, q) and np.array_equal(sT, s)
    w = qr_synth.normal_bf16(31, (200, 136), 0.02)
    qb, sb = oracle.quant_blocks(w)
    wp = np.zeros((256, 256), np.uint16)
    wp[:200, :136] = w
    qbp, sbp = oracle.quant_blocks(wp)
    assert np.array_equal(qb, qbp[:200, :136]) and np.array_equal(sb, sbp)


def test_nonfinite_input_rejected():
    x = np.zeros((1, 128), np.uint16)
    for bad in (0x7F80, 0xFF80, 0x7FC0):
        x[0, 5] = bad
        with pytest.raises(ValueError):
            oracle.quant_rows(x)
        with pytest.raises(ValueError):
            oracle.quant_blocks(x)


# ============================================================== GEMM

def _random_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38                               # no NaN codes
    return c


@pytest.mark.parametrize("K", [128, 256, 384])
def test_gemm_bruteforce_fractions(K):
    rng = np.random.default_rng(K)
    M, N = 3, 5
    qa = _random_codes(rng, (M, K))
    sa = rng.uniform(1e-3, 2.0, (M, K // 128)).astype(np.float32)
    qw = _random_codes(rng, (N, K))
    sw = rng.uniform(1e-3, 2.0, (1, K // 128)).astype(np.float32)
    Y, S = oracle.fprop(qa, sa, qw, sw)
    tv = e4m3_values_torch()
    for m in range(M):
        for n in range(N):
            y = Fraction(0)
            a = Fraction(0)
            for k in range(K):
                p = (Fraction(float(tv[qa[m, k]])) * Fraction(float(sa[m, k // 128])) *
                     Fraction(float(tv[qw[n, k]])) * Fraction(float(sw[0, k // 128])))
                y += p
                a += abs(p)
            assert abs(Fraction(Y[m, n]) - y) <= Fraction(1, 10 ** 12) * a
            assert abs(Fraction(S[m, n]) - a) <= Fraction(1, 10 ** 12) * a


def _int_codes():
    """Codes whose values are the integers -16..16 (all exact in E4M3)."""
    tv = e4m3_values_torch()
    lut = {}
    for c in range(256):
        v = tv[c]
        if not np.isnan(v) and v == int(v) and abs(v) <= 16 and int(v) not in lut:
            lut[int(v)] = c
    assert sorted(lut) == list(range(-16, 17))
    return lut


def test_gemm_integer_special_case_exact():
    lut = _int_codes()
    rng = np.random.default_rng(3)
    M, N, K = 7, 9, 256
    ia = rng.integers(-16, 17, (M, K))
    iw = rng.integers(-16, 17, (N, K))
    qa = np.vectorize(lut.get)(ia).astype(np.uint8)
    qw = np.vectorize(lut.get)(iw).astype(np.uint8)
    Y, _ = oracle.fprop(qa, np.ones((M, 2), np.float32), qw, np.ones((1, 2), np.float32))
    assert np.array_equal(Y, (ia.astype(np.int64) @ iw.T.astype(np.int64)).astype(np.float64))
    # the same integers through DGrad's and WGrad's layouts
    iw2 = rng.integers(-16, 17, (128, 9))                  # W [N=128, K=9] for DGrad
    qw2 = np.vectorize(lut.get)(iw2).astype(np.uint8)
    dX, _ = oracle.dgrad(np.ascontiguousarray(qa[:, :128]), np.ones((M, 1), np.float32), qw2,
                         np.ones((1, 1), np.float32))
    assert np.array_equal(dX, (ia[:, :128] @ iw2).astype(np.float64))
    # WGrad operands are token-grouped rows: dY^T [7, 128 tokens], X^T [9, 128 tokens]
    dW, _ = oracle.wgrad(np.ascontiguousarray(qa[:, :128]), np.ones((M, 1), np.float32),
                         np.ascontiguousarray(qw[:, :128]), np.ones((N, 1), np.float32))
    assert np.array_equal(dW, (ia[:, :128] @ iw[:, :128].T).astype(np.float64))


def test_gemm_identity_weight():
    x = qr_synth.normal_bf16(41, (64, 256), 1.0, 42, 2)
    qa, sa = oracle.quant_rows(x)
    qw = np.zeros((256, 256), np.uint8)
    np.fill_diagonal(qw, 0x38)
    Y, _ = oracle.fprop(qa, sa, qw, np.ones((2, 2), np.float32))
    assert np.array_equal(Y, oracle.dequant_rows(qa, sa))


def test_dgrad_is_fprop_with_transposed_weight():
    dy = qr_synth.normal_bf16(43, (96, 256), 1e-3)
    w = qr_synth.normal_bf16(44, (256, 384), 0.02)
    qd, sd = oracle.quant_rows(dy)
    qw, sw = oracle.quant_blocks(w)
    dX, S1 = oracle.dgrad(qd, sd, qw, sw)
    Y, S2 = oracle.fprop(qd, sd, np.ascontiguousarray(qw.T), np.ascontiguousarray(sw.T))
    assert np.allclose(dX, Y, rtol=0, atol=1e-12 * S1.max()) and np.allclose(S1, S2)


def test_gemms_against_numpy_blas():
    x = qr_synth.normal_bf16(45, (256, 384), 1.0, 46, 4)
    dy = qr_synth.normal_bf16(47, (256, 512), 1e-3)
    qxT, sxT = oracle.quant_cols_T(x)
    qdT, sdT = oracle.quant_cols_T(dy)
    dW, S = oracle.wgrad(qdT, sdT, qxT, sxT)
    A = oracle.dequant_rows(qdT, sdT)
    B = oracle.dequant_rows(qxT, sxT)
    assert dW.shape == (512, 384)
    assert np.all(np.abs(dW - A @ B.T) <= 1e-12 * S)
    assert np.allclose(S, np.abs(A) @ np.abs(B).T, rtol=1e-12)
    # sampled sums equal the full ones exactly (same loop, same order)
    mi = np.array([0, 5, 511, 100]), np.array([0, 383, 7, 200])
    Ys, Ss = oracle.wgrad(qdT, sdT, qxT, sxT, sample=mi)
    assert np.array_equal(Ys, dW[mi]) and np.array_equal(Ss, S[mi])


# ============================================================== UAQ fold

def test_uaq_golden_s1p5():
    rows = [p for p in _golden_lines("uaq_s1p5.txt")]
    wrows = [(int(a, 16), int(b, 16)) for a, b, *_ in rows if a != "gain"]
    w = np.array([[a for a, _ in wrows]], np.uint16)
    s = np.full(w.shape[1], 1.5, np.float32)
    gains = [(np.float32(r[1]), np.float32(r[2])) for r in rows if r[0] == "gain"]
    g = np.array([a for a, _ in gains] + [1.0] * (w.shape[1] - len(gains)), np.float32)
    out, g2 = oracle.uaq_fold(w, s, g)
    assert [int(v) for v in out[0]] == [b for _, b in wrows]
    for i, (_, b) in enumerate(gains):
        assert g2[i] == b


def _uaq_cases():
    """Random folds, plus near-midpoint folds: s = RN32(W / mid) for a bf16 midpoint mid puts
    W/s within about 2^-24 (relative) of mid, where rounding W/s to binary32 first and then to
    bf16 would often land on the midpoint and round the wrong way.  (An exact tie cannot
    occur: a midpoint's odd 9-bit significand cannot divide an 8-bit one.)"""
    rng = np.random.default_rng(51)
    w = qr_synth.normal_bf16(52, (16, 96), 0.02)
    s = rng.uniform(1.5, 4.0, 96).astype(np.float32)
    wb = qr_synth.normal_bf16(60, (1, 400), 0.02)[0]
    wv = bf16_f32(wb).astype(np.float64)
    # a midpoint below |W|/1.5 so that s lands in the UAQ range (>= 1.5)
    mids = []
    for v in wv:
        tgt = abs(v) / rng.uniform(1.5, 4.0)
        e = math.floor(math.log2(tgt))
        ulp = 2.0 ** (e - 7)
        mids.append((math.floor(tgt / ulp) + 0.5) * ulp)
    ms = np.array([abs(v) / m for v, m in zip(wv, mids)], np.float32)
    return w, s, wb[None, :], ms


def test_uaq_matches_exact_rational_rounding():
    w, s, mw, ms = _uaq_cases()
    naive_wrong = 0
    for W, S in ((w, s), (mw, ms)):
        out, _ = oracle.uaq_fold(W, S)
        for (i, j), b in np.ndenumerate(W):
            q = Fraction(float(bf16_f32(np.uint16(b)).item())) / Fraction(float(S[j]))
            assert int(out[i, j]) & 0x7FFF == bf16_bits_of(abs(rn_bf16(q))), (hex(b), S[j])
            assert (int(out[i, j]) >> 15) == (int(b) >> 15)
            if W is mw:
                naive = rn_bf16(rn32(q))
                naive_wrong += naive != rn_bf16(q)
    assert naive_wrong > 20          # the near-midpoint set does exercise double rounding


def test_uaq_power_of_two_and_identity():
    w = qr_synth.normal_bf16(53, (32, 256), 0.02)
    out, _ = oracle.uaq_fold(w, np.ones(256, np.float32))
    assert np.array_equal(out, w)
    out, _ = oracle.uaq_fold(w, np.full(256, 4.0, np.float32))
    assert np.array_equal(bf16_f32(out), bf16_f32(w) / np.float32(4.0))   # exact shift
    # s = 2^j then 128x128 quantization: same codes, block scales divided by 2^j
    q0, s0 = oracle.quant_blocks(w)
    q1, s1 = oracle.quant_blocks(out)
    assert np.array_equal(q0, q1) and np.array_equal(s1, s0 / np.float32(4.0))


def test_uaq_preserves_product_exactly_before_rounding_and_within_bf16_after():
    """WX = (W/s)(sX): exact in rationals; after the bf16 rounding of W/s the product moves
    by at most 2^-8 * sum |W X| per output."""
    rng = np.random.default_rng(55)
    w = qr_synth.normal_bf16(56, (4, 128), 0.02)
    x = qr_synth.normal_bf16(57, (3, 128), 1.0)
    s = rng.uniform(1.5, 4.0, 128).astype(np.float32)
    wf, xf = bf16_f32(w), bf16_f32(x)
    out, _ = oracle.uaq_fold(w, s)
    of = bf16_f32(out)
    for n in range(4):
        for m in range(3):
            exact = sum(Fraction(float(wf[n, k])) * Fraction(float(xf[m, k])) for k in range(128))
            folded = sum((Fraction(float(wf[n, k])) / Fraction(float(s[k]))) *
                         (Fraction(float(s[k])) * Fraction(float(xf[m, k]))) for k in range(128))
            assert folded == exact
            rounded = sum(Fraction(float(of[n, k])) * Fraction(float(s[k])) *
                          Fraction(float(xf[m, k])) for k in range(128))
            bound = Fraction(1, 256) * sum(abs(Fraction(float(wf[n, k])) * Fraction(float(xf[m, k])))
                                           for k in range(128))
            assert abs(rounded - exact) <= bound


def test_uaq_gain_and_rejections():
    rng = np.random.default_rng(59)
    s = rng.uniform(1.5, 4.0, 128).astype(np.float32)
    g = rng.uniform(0.5, 2.0, 128).astype(np.float32)
    _, g2 = oracle.uaq_fold(np.zeros((1, 128), np.uint16), s, g)
    assert np.array_equal(g2, (g * s).astype(np.float32))
    for i in range(0, 128, 17):
        assert Fraction(float(g2[i])) == rn32(Fraction(float(g[i])) * Fraction(float(s[i])))
    bad = s.copy()
    bad[3] = 0.0
    with pytest.raises(ValueError):
        oracle.uaq_fold(np.zeros((1, 128), np.uint16), bad)


# ============================================================== RMSNorm (the norm carrying s)

def _bf16_frac(b):
    return Fraction(float(bf16_f32(np.array([b], np.uint16))[0]))


def _exact_rms_bf16(hrow, grow, eps):
    """RN_bf16(h * g / sqrt(q)), q = mean(h^2) + eps, decided in exact rationals: for a
    candidate bf16 bracket lo <= |y| < hi (from a float estimate, verified exactly), |y| lies
    above the midpoint m iff (h g)^2 > m^2 q.  Returns bf16 bit patterns."""
    hv = [Fraction(float(v)) for v in hrow]
    q = sum(v * v for v in hv) / len(hv) + Fraction(float(np.float32(eps)))
    out = []
    for v, g in zip(hv, grow):
        a2 = (v * Fraction(float(g))) ** 2 / q          # y^2, exact
        sign = (v * Fraction(float(g))) < 0
        if a2 == 0:
            out.append(0x8000 if sign else 0)
            continue
        est = math.sqrt(float(a2))
        b = int(np.array([est], np.float32).view(np.uint32)[0]) >> 16   # truncated estimate
        for _ in range(4):                                # move the bracket until it holds
            lo, hi = _bf16_frac(b), _bf16_frac(b + 1)
            if lo * lo > a2:
                b -= 1
            elif hi * hi <= a2:
                b += 1
            else:
                break
        lo, hi = _bf16_frac(b), _bf16_frac(b + 1)
        assert lo * lo <= a2 < hi * hi
        mid2 = ((lo + hi) / 2) ** 2
        up = a2 > mid2 or (a2 == mid2 and (b & 1))
        out.append((b + up) | (0x8000 if sign else 0))
    return out


def test_rmsnorm_matches_exact_rational_rounding():
    rng = np.random.default_rng(71)
    for i, (std, eps) in enumerate([(1.0, 1e-6), (1e-3, 1e-6), (30.0, 0.0), (0.05, 1.0)]):
        h = qr_synth.normal_bf16(72 + i, (3, 96), std, 73 + i, 2)
        g = rng.uniform(0.5, 4.0, 96).astype(np.float32)
        g[::7] *= -1.0
        _, yb = oracle.rmsnorm(h, g, eps)
        hf = bf16_f32(h)
        for r in range(h.shape[0]):
            assert [int(v) for v in yb[r]] == _exact_rms_bf16(hf[r], g, eps), (std, eps, r)


def test_rmsnorm_constant_rows_and_power_of_two_invariance():
    # a constant row with eps = 0 normalizes to +-1 exactly (times the gain)
    vals = [0x3F80, 0x4049, 0xC2F7, 0x0123, 0x7F00, 0xB8A1]
    h = np.array([[v] * 256 for v in vals], np.uint16)
    y, yb = oracle.rmsnorm(h, np.ones(256, np.float32), 0.0)
    for r, v in enumerate(vals):
        assert np.all(yb[r] == (0xBF80 if v & 0x8000 else 0x3F80)), hex(v)
    # scaling h by 2^j leaves y unchanged when eps = 0
    h = qr_synth.normal_bf16(75, (8, 512), 1.0, 76, 5)
    g = np.random.default_rng(77).uniform(0.5, 2.0, 512).astype(np.float32)
    y0, b0 = oracle.rmsnorm(h, g, 0.0)
    h8 = qr_synth.f32_to_bf16_bits(bf16_f32(h) * np.float32(2.0 ** -20))
    y1, b1 = oracle.rmsnorm(h8, g, 0.0)
    assert np.array_equal(b0, b1) and np.array_equal(y0, y1)


def test_rmsnorm_rejections():
    h = np.zeros((2, 128), np.uint16)
    g = np.ones(128, np.float32)
    with pytest.raises(ValueError):
        oracle.rmsnorm(h, g, -1.0)
    bad = g.copy()
    bad[5] = np.inf
    with pytest.raises(ValueError):
        oracle.rmsnorm(h, bad, 1e-6)
    h[1, 3] = 0x7F80
    with pytest.raises(ValueError):
        oracle.rmsnorm(h, g, 1e-6)


# ============================================================== INT8 W8A8 variant

def test_int8_rows_match_exact_rationals():
    """s = RN32(amax / 127) and q = clamp(RNE(RN32(x / s)), +-127), decided in rationals
    (Python rounds Fractions half to even)."""
    for seed, std in ((81, 1.0), (83, 1e-3), (85, 3e4)):
        x = qr_synth.normal_bf16(seed, (5, 200), std, seed + 1, 3)
        q, s = oracle.quant_int8_rows(x)
        xf = bf16_f32(x)
        for r in range(5):
            amax = max(abs(Fraction(float(v))) for v in xf[r])
            sr = rn32(amax / 127)
            assert Fraction(float(s[r])) == sr
            for c in range(200):
                n = round(rn32(Fraction(float(xf[r, c])) / sr))
                assert int(q[r, c]) == max(-127, min(127, n)), (seed, r, c)


def test_int8_ties_amax_zero_and_symmetries():
    # amax = 127 gives s = 1 exactly, so x = k + 1/2 is an exact tie: to even
    row = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0]
    x = qr_synth.f32_to_bf16_bits(np.array([row + [0.0] * 6], np.float32))
    q, s = oracle.quant_int8_rows(x)
    assert s[0] == 1.0
    assert [int(v) for v in q[0, :10]] == [127, 2, 4, -2, -4, 0, 0, 2, 126, -127]
    # the amax element of any row encodes to +-127; a zero row has s = 0 and zero codes
    x = qr_synth.normal_bf16(87, (64, 96), 1.0)
    x[5] = 0
    q, s = oracle.quant_int8_rows(x)
    amax_pos = np.argmax(np.abs(bf16_f32(x)), axis=1)
    for r in range(64):
        if r == 5:
            assert s[r] == 0 and not q[r].any()
        else:
            assert abs(int(q[r, amax_pos[r]])) == 127
    # sign symmetry and power-of-two invariance
    qn, sn = oracle.quant_int8_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    x2 = qr_synth.f32_to_bf16_bits(bf16_f32(x) * np.float32(2.0 ** 40))
    q2, s2 = oracle.quant_int8_rows(x2)
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** 40))
    # error bound: |x - q s| <= s (1/2 + 127 * 2^-24): half a step, plus the binary32
    # quotient's own rounding (relative 2^-24 of |x/s| <= 127)
    err = np.abs(bf16_f32(x).astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -24))


def test_int8_gemm_brute_force():
    rng = np.random.default_rng(89)
    for M, N, K in ((3, 5, 128), (4, 4, 256), (2, 7, 384)):
        qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
        qb = rng.integers(-127, 128, (N, K)).astype(np.int8)
        sa = rng.uniform(1e-3, 2.0, M).astype(np.float32)
        sb = rng.uniform(1e-3, 2.0, N).astype(np.float32)
        Y = oracle.gemm_int8(qa, sa, qb, sb)
        for m in range(M):
            for n in range(N):
                acc = sum(int(qa[m, k]) * int(qb[n, k]) for k in range(K))
                exact = Fraction(float(sa[m])) * Fraction(float(sb[n])) * acc
                assert abs(Fraction(float(Y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
        mi, ni = np.array([0, M - 1, 1]), np.array([N - 1, 0, 2])
        assert np.array_equal(oracle.gemm_int8(qa, sa, qb, sb, sample=(mi, ni)), Y[mi, ni])


# ============================================================== 4-bit (NVFP4-style) weights

E2M1_HAND = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]          # 1 sign, 2 exponent (bias 1), 1 mantissa


def _e2m1_nearest(v: Fraction):
    """Nearest E2M1 code by search, ties to the even code, saturating at 6 (sign kept)."""
    sign = 8 if v < 0 else 0
    a = abs(v)
    best = min(range(8), key=lambda c: (abs(a - Fraction(E2M1_HAND[c])), c & 1))
    return sign | best


def test_e2m1_codec_hand_values_midpoints_and_saturation():
    for c in range(16):
        v = E2M1_HAND[c & 7] * (-1 if c & 8 else 1)
        assert oracle.lib().orc_e2m1_decode(c) == v
        if c != 8:
            assert oracle.lib().orc_e2m1_encode(v) == c              # round trip
    assert oracle.lib().orc_e2m1_encode(-0.0) == 8                   # sign of zero kept
    mids = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for m, code in mids:                                              # ties to the even code
        assert oracle.lib().orc_e2m1_encode(m) == code, m
        assert oracle.lib().orc_e2m1_encode(-m) == 8 | code
        assert oracle.lib().orc_e2m1_encode(np.nextafter(np.float32(m), np.float32(9))) == \
            _e2m1_nearest(Fraction(float(np.nextafter(np.float32(m), np.float32(9)))))
        assert oracle.lib().orc_e2m1_encode(np.nextafter(np.float32(m), np.float32(0))) == \
            _e2m1_nearest(Fraction(float(np.nextafter(np.float32(m), np.float32(0)))))
    for v in (6.0, 6.5, 100.0, 3.0e38):                              # saturation
        assert oracle.lib().orc_e2m1_encode(v) == 7 and oracle.lib().orc_e2m1_encode(-v) == 15


def test_nvfp4_quantizer_matches_exact_rationals():
    """t = RN32(amax / 2688), u = RN32(6 t), block scale = E4M3(RN32(amax_b / u)),
    e = RN32(dq(scale) t), code = E2M1(RN32(x / e)), all decided in rationals with searches."""
    for seed, std in ((91, 0.02), (93, 1.0), (95, 3e-3)):
        w = qr_synth.normal_bf16(seed, (6, 64), std, seed + 1, 2)
        codes, bs, t = oracle.quant_nvfp4(w)
        wf = bf16_f32(w)
        amax = max(abs(Fraction(float(v))) for v in wf.ravel())
        tr = rn32(amax / 2688)
        assert Fraction(t) == tr
        u = rn32(6 * tr)
        vals = e4m3_values_torch()
        for r in range(6):
            for b in range(4):
                blk = [Fraction(float(v)) for v in wf[r, 16 * b:16 * b + 16]]
                sb = e4m3_nearest(float(rn32(max(abs(v) for v in blk) / u)))
                assert int(bs[r, b]) == sb
                e = rn32(Fraction(float(vals[sb])) * tr)
                for j, v in enumerate(blk):
                    c = 16 * b + j
                    got = (int(codes[r, c // 2]) >> (4 * (c & 1))) & 15
                    want = _e2m1_nearest(rn32(v / e)) if e != 0 else (8 if v < 0 else 0)
                    if v == 0:
                        want = 8 if np.signbit(wf[r, c]) else 0
                    assert got == want, (seed, r, c)


def test_nvfp4_amax_element_zero_weight_and_power_of_two():
    w = qr_synth.normal_bf16(97, (8, 128), 0.02)
    codes, bs, t = oracle.quant_nvfp4(w)
    wf = bf16_f32(w)
    r, c = np.unravel_index(np.argmax(np.abs(wf)), wf.shape)
    assert bs[r, c // 16] == 0x7E                                     # block scale 448
    assert (int(codes[r, c // 2]) >> (4 * (c & 1))) & 7 == 7          # code +-6
    z = np.zeros((4, 32), np.uint16)
    z[1, 3] = 0x8000
    cz, bz, tz = oracle.quant_nvfp4(z)
    assert tz == 0 and not bz.any()
    assert ((cz[1, 1] >> 4) & 15) == 8 and (cz & 0x77).sum() == 0     # signed zeros only
    w2 = qr_synth.f32_to_bf16_bits(wf * np.float32(2.0 ** 30))
    c2, b2, t2 = oracle.quant_nvfp4(w2)
    assert np.array_equal(c2, codes) and np.array_equal(b2, bs) and t2 == t * 2.0 ** 30


def test_w4a16_gemm_brute_force():
    rng = np.random.default_rng(99)
    w = qr_synth.normal_bf16(100, (5, 96), 0.02)
    x = qr_synth.normal_bf16(101, (3, 96), 1.0)
    codes, bs, t = oracle.quant_nvfp4(w)
    Y = oracle.gemm_w4a16(x, codes, bs, t)
    vals = e4m3_values_torch()
    xf = bf16_f32(x)
    for m in range(3):
        for n in range(5):
            acc = Fraction(0)
            for k in range(96):
                code = (int(codes[n, k // 2]) >> (4 * (k & 1))) & 15
                wv = Fraction(E2M1_HAND[code & 7]) * (-1 if code & 8 else 1) * \
                    Fraction(float(vals[bs[n, k // 16]]))
                acc += Fraction(float(xf[m, k])) * wv
            exact = acc * Fraction(t)
            assert abs(Fraction(float(Y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 48) + \
                Fraction(1, 2 ** 120)
    mi, ni = np.array([0, 2, 1]), np.array([4, 0, 3])
    assert np.array_equal(oracle.gemm_w4a16(x, codes, bs, t, sample=(mi, ni)), Y[mi, ni])
