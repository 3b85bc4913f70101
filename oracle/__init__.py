"""Reference oracle for the fine-grained FP8 quantize-and-multiply path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It shares no code with the HIP library and never imports it.  All arrays are numpy
arrays on the host: bf16 tensors are passed as their uint16 bit patterns.

The arithmetic lives in ``qr_oracle.c`` (plain scalar C, fp64 products); this module only
marshals arguments and strings the definitions together:

* ``quant_rows``   -- 1x128 groups along rows (activations, gradients).
* ``quant_cols_T`` -- 128x1 groups down columns, stored transposed (WGrad's operands).
* ``quant_blocks`` -- 128x128 blocks (weights).
* ``fprop`` / ``dgrad`` / ``wgrad`` -- dequantize, then multiply in fp64 (returns Y and
  S = sum |a*b|, the quantity the GEMM tolerance is stated against).
* ``uaq_fold``     -- W' = RN_bf16(W / s[col]), gain' = RN32(gain * s).
* ``quant_nvfp4`` / ``gemm_w4a16`` -- the 4-bit weight path (E2M1 elements, E4M3 scales per
  16, an fp32 tensor scale) and its bf16-activation GEMM.
* ``quant_int8_rows`` / ``gemm_int8`` -- the INT8 W8A8 variant (one symmetric scale per row,
  exact integer products).
* ``rmsnorm``      -- the norm whose gain carries the UAQ scale: y = h * gain / sqrt(mean(h^2)
  + eps) in fp64 and its RN_bf16 (the input of the fused norm-and-quantize kernel).

Sources: Jet-RL (arXiv 2601.14243v1) notes, section on the fine-grained GEMM quantization
scheme (Figure 6 there); QuRL (ICLR 2026) notes, key design 1 (UAQ).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64

GROUP = 128


def lib():
    """Load (building first if absent or stale) the compiled oracle."""
    global _LIB
    if _LIB is None:
        src_m = os.path.getmtime(_build.SRC)
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < src_m:
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_group_scale.argtypes = [ctypes.c_float]
        L.orc_group_scale.restype = ctypes.c_float
        L.orc_quantize_value.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_quantize_value.restype = ctypes.c_uint8
        L.orc_e4m3_encode_array.argtypes = [_f32p, _i64, _u8p]
        L.orc_e4m3_encode_array.restype = None
        L.orc_quantize_value_array.argtypes = [_f32p, _f32p, _i64, _u8p]
        L.orc_quantize_value_array.restype = None
        for name in ("orc_quant_rows_1x128", "orc_quant_cols_128x1_T", "orc_quant_blocks_128x128"):
            f = getattr(L, name)
            f.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _f32p]
            f.restype = ctypes.c_int
        L.orc_dequant_rows.argtypes = [_u8p, _f32p, _i64, _i64, _f64p]
        L.orc_dequant_rows.restype = None
        L.orc_dequant_blocks.argtypes = [_u8p, _f32p, _i64, _i64, _f64p]
        L.orc_dequant_blocks.restype = None
        L.orc_matmul_nt.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _f64p, _f64p]
        L.orc_matmul_nt.restype = None
        L.orc_matmul_nt_sampled.argtypes = [_f64p, _f64p, _i64, _i64p, _i64p, _i64, _f64p, _f64p]
        L.orc_matmul_nt_sampled.restype = None
        L.orc_uaq_fold.argtypes = [_u16p, _i64, _i64, _i64, _f32p, _u16p, _f32p]
        L.orc_uaq_fold.restype = ctypes.c_int
        L.orc_rmsnorm.argtypes = [_u16p, _i64, _i64, _i64, _f32p, ctypes.c_float, _f64p, _u16p]
        L.orc_rmsnorm.restype = ctypes.c_int
        _i8p = ctypes.POINTER(ctypes.c_int8)
        L.orc_quant_int8_rows.argtypes = [_u16p, _i64, _i64, _i64, _i8p, _f32p]
        L.orc_quant_int8_rows.restype = ctypes.c_int
        L.orc_gemm_int8.argtypes = [_i8p, _f32p, _i8p, _f32p, _i64, _i64, _i64, _f64p]
        L.orc_gemm_int8.restype = None
        L.orc_gemm_int8_sampled.argtypes = [_i8p, _f32p, _i8p, _f32p, _i64, _i64p, _i64p, _i64,
                                            _f64p]
        L.orc_gemm_int8_sampled.restype = None
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_encode.argtypes = [ctypes.c_float]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_quant_nvfp4.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _u8p, _f32p]
        L.orc_quant_nvfp4.restype = ctypes.c_int
        L.orc_gemm_w4a16.argtypes = [_u16p, _u8p, _u8p, ctypes.c_float, _i64, _i64, _i64, _i64p,
                                     _i64p, _i64, _f64p]
        L.orc_gemm_w4a16.restype = None
        _LIB = L
    return _LIB


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def ngroups(n: int) -> int:
    return (n + GROUP - 1) // GROUP


# ------------------------------------------------------------------ scalar codec

def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(v)))


def e4m3_decode_table() -> np.ndarray:
    """Exact value of every code 0..255 (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32).ravel())
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(v, _f32p), v.size, _p(out, _u8p))
    return out


def quantize_value_array(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes of elements x given their group scales s (same shape)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float32).ravel())
    assert x.shape == s.shape
    out = np.empty(x.shape, np.uint8)
    lib().orc_quantize_value_array(_p(x, _f32p), _p(s, _f32p), x.size, _p(out, _u8p))
    return out


def group_scale(amax: float) -> np.float32:
    return np.float32(lib().orc_group_scale(float(np.float32(amax))))


def quantize_value(x: float, s: float) -> int:
    return int(lib().orc_quantize_value(float(np.float32(x)), float(np.float32(s))))


# ------------------------------------------------------------------ quantizers

def quant_rows(x_bf16: np.ndarray):
    """1x128 groups along each row of a [rows, cols] bf16 tensor -> (q u8 [rows, cols],
    s f32 [rows, ceil(cols/128)])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, ngroups(cols)), np.float32)
    if lib().orc_quant_rows_1x128(_p(x, _u16p), rows, cols, cols, _p(q, _u8p), _p(s, _f32p)):
        raise ValueError("non-finite input to the 1x128 quantizer")
    return q, s


def quant_cols_T(x_bf16: np.ndarray):
    """128x1 groups down each column of a [rows, cols] bf16 tensor, stored transposed ->
    (qT u8 [cols, rows], sT f32 [cols, ceil(rows/128)])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    qT = np.empty((cols, rows), np.uint8)
    sT = np.empty((cols, ngroups(rows)), np.float32)
    if lib().orc_quant_cols_128x1_T(_p(x, _u16p), rows, cols, cols, _p(qT, _u8p), _p(sT, _f32p)):
        raise ValueError("non-finite input to the 128x1 quantizer")
    return qT, sT


def quant_blocks(w_bf16: np.ndarray):
    """128x128 blocks of a [n, k] bf16 weight -> (q u8 [n, k], s f32 [ceil(n/128), ceil(k/128)]).
    The transposed copy for DGrad is (q.T, s.T)."""
    w = _c(w_bf16, np.uint16)
    n, k = w.shape
    q = np.empty((n, k), np.uint8)
    s = np.empty((ngroups(n), ngroups(k)), np.float32)
    if lib().orc_quant_blocks_128x128(_p(w, _u16p), n, k, k, _p(q, _u8p), _p(s, _f32p)):
        raise ValueError("non-finite input to the 128x128 quantizer")
    return q, s


def dequant_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    rows, cols = q.shape
    assert s.shape == (rows, ngroups(cols))
    out = np.empty((rows, cols), np.float64)
    lib().orc_dequant_rows(_p(q, _u8p), _p(s, _f32p), rows, cols, _p(out, _f64p))
    return out


def dequant_blocks(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    n, k = q.shape
    assert s.shape == (ngroups(n), ngroups(k))
    out = np.empty((n, k), np.float64)
    lib().orc_dequant_blocks(_p(q, _u8p), _p(s, _f32p), n, k, _p(out, _f64p))
    return out


# ------------------------------------------------------------------ products

def matmul_nt(A: np.ndarray, B: np.ndarray):
    """Y = A @ B.T and S = |A| @ |B|.T elementwise sums, fp64, plain loops."""
    A = _c(A, np.float64)
    B = _c(B, np.float64)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    lib().orc_matmul_nt(_p(A, _f64p), _p(B, _f64p), M, N, K, _p(Y, _f64p), _p(S, _f64p))
    return Y, S


def matmul_nt_sampled(A: np.ndarray, B: np.ndarray, mi: np.ndarray, ni: np.ndarray):
    A = _c(A, np.float64)
    B = _c(B, np.float64)
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    K = A.shape[1]
    assert B.shape[1] == K and mi.shape == ni.shape
    assert mi.size == 0 or (mi.min() >= 0 and mi.max() < A.shape[0])
    assert ni.size == 0 or (ni.min() >= 0 and ni.max() < B.shape[0])
    Y = np.empty(mi.shape, np.float64)
    S = np.empty(mi.shape, np.float64)
    lib().orc_matmul_nt_sampled(_p(A, _f64p), _p(B, _f64p), K, _p(mi, _i64p), _p(ni, _i64p),
                                mi.size, _p(Y, _f64p), _p(S, _f64p))
    return Y, S


def fprop(qa, sa, qw, sw, sample=None):
    """Y[m, n] = sum_k deq(A)[m, k] deq(W)[n, k]; A 1x128 along K, W 128x128.
    ``sample`` = (mi, ni) restricts the sums to those output positions."""
    A = dequant_rows(qa, sa)
    B = dequant_blocks(qw, sw)
    return matmul_nt(A, B) if sample is None else matmul_nt_sampled(A, B, *sample)


def dgrad(qdy, sdy, qw, sw, sample=None):
    """dX[m, k] = sum_n deq(dY)[m, n] deq(W)[n, k]; dY 1x128 along N, W 128x128 [N, K]."""
    A = dequant_rows(qdy, sdy)
    Bt = np.ascontiguousarray(dequant_blocks(qw, sw).T)    # [K, N]
    return matmul_nt(A, Bt) if sample is None else matmul_nt_sampled(A, Bt, *sample)


def wgrad(qdyT, sdyT, qxT, sxT, sample=None):
    """dW[n, k] = sum_m deq(dY)[m, n] deq(X)[m, k] with both operands grouped 128 along the
    token index m; inputs are the transposed outputs of ``quant_cols_T`` (dY^T [N, M],
    X^T [K, M]), whose groups run along their rows."""
    A = dequant_rows(qdyT, sdyT)   # dY^T values [N, M]
    B = dequant_rows(qxT, sxT)     # X^T values  [K, M]
    return matmul_nt(A, B) if sample is None else matmul_nt_sampled(A, B, *sample)


# ------------------------------------------------------------------ UAQ

def uaq_fold(w_bf16: np.ndarray, s: np.ndarray, gain=None):
    """Returns (W' bf16 bits [n, k], gain' f32 [k] or None)."""
    w = _c(w_bf16, np.uint16)
    n, k = w.shape
    s = _c(np.asarray(s), np.float32)
    assert s.shape == (k,)
    out = np.empty_like(w)
    g = None if gain is None else _c(np.asarray(gain, np.float32).copy(), np.float32)
    rc = lib().orc_uaq_fold(_p(w, _u16p), n, k, k, _p(s, _f32p), _p(out, _u16p),
                            None if g is None else _p(g, _f32p))
    if rc:
        raise ValueError("UAQ fold: non-finite weight or non-positive scale")
    return out, g


# ------------------------------------------------------------------ RMSNorm

def rmsnorm(h_bf16: np.ndarray, gain: np.ndarray, eps: float):
    """Returns (y fp64 [rows, cols], RN_bf16(y) bits [rows, cols]) for
    y = h * gain / sqrt(mean(h^2 over the row) + eps)."""
    h = _c(h_bf16, np.uint16)
    rows, cols = h.shape
    g = _c(np.asarray(gain, np.float32), np.float32)
    assert g.shape == (cols,)
    y = np.empty((rows, cols), np.float64)
    yb = np.empty((rows, cols), np.uint16)
    if lib().orc_rmsnorm(_p(h, _u16p), rows, cols, cols, _p(g, _f32p), float(eps), _p(y, _f64p),
                         _p(yb, _u16p)):
        raise ValueError("RMSNorm: non-finite input or gain, or a bad eps")
    return y, yb


# ------------------------------------------------------------------ INT8 W8A8

_i8p = ctypes.POINTER(ctypes.c_int8)


def quant_int8_rows(x_bf16: np.ndarray):
    """One symmetric INT8 scale per row of a [rows, cols] bf16 tensor -> (q int8 [rows, cols],
    s f32 [rows])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    if lib().orc_quant_int8_rows(_p(x, _u16p), rows, cols, cols, _p(q, _i8p), _p(s, _f32p)):
        raise ValueError("non-finite input to the INT8 quantizer")
    return q, s


def gemm_int8(qa, sa, qb, sb, sample=None):
    """Y = sa[m] sb[n] sum_k qa[m, k] qb[n, k] (exact integer sum, fp64 scaling); with
    sample=(mi, ni) only those positions."""
    A, B = _c(qa, np.int8), _c(qb, np.int8)
    M, K = A.shape
    N = B.shape[0]
    sa, sb = _c(np.asarray(sa), np.float32), _c(np.asarray(sb), np.float32)
    if sample is None:
        Y = np.empty((M, N), np.float64)
        lib().orc_gemm_int8(_p(A, _i8p), _p(sa, _f32p), _p(B, _i8p), _p(sb, _f32p), M, N, K,
                            _p(Y, _f64p))
        return Y
    mi, ni = (_c(np.asarray(v), np.int64) for v in sample)
    Y = np.empty(mi.size, np.float64)
    lib().orc_gemm_int8_sampled(_p(A, _i8p), _p(sa, _f32p), _p(B, _i8p), _p(sb, _f32p), K,
                                _p(mi, _i64p), _p(ni, _i64p), mi.size, _p(Y, _f64p))
    return Y


# ------------------------------------------------------------------ 4-bit weights

def quant_nvfp4(w_bf16: np.ndarray):
    """[n, k] bf16 weight (k % 16 == 0) -> (codes u8 [n, k/2], block scales u8 [n, k/16] (E4M3
    codes), tensor scale float)."""
    w = _c(w_bf16, np.uint16)
    n, k = w.shape
    codes = np.empty((n, k // 2), np.uint8)
    bs = np.empty((n, k // 16), np.uint8)
    t = np.zeros(1, np.float32)
    if lib().orc_quant_nvfp4(_p(w, _u16p), n, k, k, _p(codes, _u8p), _p(bs, _u8p), _p(t, _f32p)):
        raise ValueError("4-bit quantizer: non-finite input or k % 16 != 0")
    return codes, bs, float(t[0])


def gemm_w4a16(x_bf16, codes, bscale, t, sample=None):
    """Y = t * X . dequant(W)^T in fp64; with sample=(mi, ni) only those positions."""
    X = _c(x_bf16, np.uint16)
    M, K = X.shape
    C, B = _c(codes, np.uint8), _c(bscale, np.uint8)
    N = C.shape[0]
    if sample is None:
        Y = np.empty((M, N), np.float64)
        lib().orc_gemm_w4a16(_p(X, _u16p), _p(C, _u8p), _p(B, _u8p), float(t), M, N, K, None,
                             None, 0, _p(Y, _f64p))
        return Y
    mi, ni = (_c(np.asarray(v), np.int64) for v in sample)
    Y = np.empty(mi.size, np.float64)
    lib().orc_gemm_w4a16(_p(X, _u16p), _p(C, _u8p), _p(B, _u8p), float(t), M, N, K,
                         _p(mi, _i64p), _p(ni, _i64p), mi.size, _p(Y, _f64p))
    return Y
