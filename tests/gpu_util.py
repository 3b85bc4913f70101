"""Helpers for the GPU parity tests: device transfer of the seeded inputs and the tolerance
check of the GEMMs against the oracle (test code only)."""
import numpy as np
import torch

import oracle
import qr_synth

GEMM_TOL = 2e-3    # |gpu - oracle| <= GEMM_TOL * sum_k |a_k b_k| per output element


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> bf16 tensor on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def assert_bitexact(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.dtype == np.float32:
        g, r = gpu.view(np.uint32), ref.view(np.uint32)
    else:
        g, r = gpu, ref
    bad = np.flatnonzero(g.ravel() != r.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ; first at flat index "
                           f"{bad[:5].tolist()}: gpu {g.ravel()[bad[:5]].tolist()} "
                           f"oracle {r.ravel()[bad[:5]].tolist()}")


def assert_gemm_close(gpu: np.ndarray, Y: np.ndarray, S: np.ndarray, what: str,
                      bf16_out: bool = False, literal: bool = False):
    """Element-wise |gpu - Y| <= GEMM_TOL * S against the unrounded fp64 oracle Y.

    The tolerance covers the fp32 accumulation.  A bf16 output adds one more rounding of that
    fp32 value y (nearest even, at most 2^-8 |y| with |y| <= |Y| + GEMM_TOL * S), which on its
    own can exceed GEMM_TOL * S wherever |Y| / S > ~0.5; for bf16 outputs that rounding is
    added to the bound, unless `literal` asks for the bare GEMM_TOL * S (the named workloads,
    whose |Y| / S stays far below 0.5).  Returns (max err/S, max |Y|/S)."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == Y.shape == S.shape, (what, gpu.shape, Y.shape)
    assert np.all(np.isfinite(gpu)), what
    err = np.abs(gpu - Y)
    lim = GEMM_TOL * S
    if bf16_out and not literal:
        lim = lim + 2.0 ** -8 * (np.abs(Y) + GEMM_TOL * S)
    bad = np.flatnonzero(err.ravel() > lim.ravel())
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(S > 0, err / S, np.where(err > 0, np.inf, 0.0))
        ys = np.where(S > 0, np.abs(Y) / S, 0.0)
    assert bad.size == 0, (f"{what}: {bad.size} of {gpu.size} outside tolerance; worst err/S "
                           f"{rel.max():.3e} at {np.unravel_index(np.argmax(rel), rel.shape)}")
    return float(rel.max()) if rel.size else 0.0, float(ys.max()) if ys.size else 0.0


def check_norm_y(yg, h, g, eps):
    """The GPU's y against the oracle's RMSNorm: equal, or one bf16 ulp off where the exact
    value lies within 2^-17 (relative) of a bf16 midpoint, plus 2^-149 where the binary32
    product is subnormal (its rounding there is absolute, up to 2^-150)."""
    yx, yb = oracle.rmsnorm(h, g, eps)
    diff = yg.astype(np.int32) - yb.astype(np.int32)
    bad = np.argwhere(diff != 0)
    assert np.all(np.abs(diff) <= 1), "y off by more than one bf16 ulp"
    for i, j in bad[:2000]:
        lo, hi = sorted((int(yg[i, j]) & 0x7FFF, int(yb[i, j]) & 0x7FFF))
        mid = (float(qr_synth.bf16_bits_to_f32(np.array([lo], np.uint16))[0]) +
               float(qr_synth.bf16_bits_to_f32(np.array([hi], np.uint16))[0])) / 2
        assert abs(abs(yx[i, j]) - mid) <= 2.0 ** -17 * abs(yx[i, j]) + 2.0 ** -149, (i, j, yx[i, j])
    assert bad.shape[0] <= max(2, yg.size // 500)


def check_w4a16(y, Y, S):
    """fp32 accumulation of K exact products: |y - Y| <= K 2^-23 sum |x w| t, plus the output
    rounding (bf16: 2^-8 |Y|)."""
    err = np.abs(y - Y)
    assert np.all(err <= S + 2.0 ** -8 * np.abs(Y) + 1e-30), float(np.max(err / (S + 1e-30)))


def sample_positions(M, N, count, seed, tile=128):
    """Output positions for sampled checks: random ones plus every row and column that sits
    on a 128-tile edge or the ragged end, paired with random partners."""
    rng = np.random.default_rng(seed)
    mi = [rng.integers(0, M, count)]
    ni = [rng.integers(0, N, count)]
    edges_m = sorted({v for b in range(0, M, tile) for v in (b, b + tile - 1, b + 63, b + 64)
                      if v < M} | {M - 1})
    edges_n = sorted({v for b in range(0, N, tile) for v in (b, b + tile - 1, b + 63, b + 64)
                      if v < N} | {N - 1})
    em = np.array(edges_m[:: max(1, len(edges_m) // 256)])
    en = np.array(edges_n[:: max(1, len(edges_n) // 256)])
    mi.append(em)
    ni.append(rng.integers(0, N, em.size))
    mi.append(rng.integers(0, M, en.size))
    ni.append(en)
    return np.concatenate(mi).astype(np.int64), np.concatenate(ni).astype(np.int64)


# ------------------------------------------------------------------ guarded outputs

GUARD = 4096          # bytes of pattern before and after every output buffer
GUARD_BYTE = 0xA5     # also the initial content of the output itself, so an element the
                      # kernel never writes cannot pass a bit-exact comparison by chance


def guarded_empty(shape, dtype, checks):
    """An output tensor inside a larger buffer whose guard bands (and body) hold GUARD_BYTE;
    appends a closure to `checks` that asserts the bands are untouched."""
    shape = tuple(int(d) for d in shape)
    elem = torch.empty((), dtype=dtype).element_size()
    nbytes = int(np.prod(shape, dtype=np.int64)) * elem
    raw = torch.full((nbytes + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device="cuda:0")
    body = raw[GUARD:GUARD + nbytes]
    t = body.view(dtype).view(shape) if nbytes else torch.empty(shape, dtype=dtype, device="cuda:0")

    def check(what="output"):
        torch.cuda.synchronize()
        lo = raw[:GUARD].cpu().numpy()
        hi = raw[GUARD + nbytes:].cpu().numpy()
        assert np.all(lo == GUARD_BYTE), f"{what} {shape}: write before the buffer"
        assert np.all(hi == GUARD_BYTE), f"{what} {shape}: write past the buffer"

    checks.append(check)
    return t


def _run_checks(checks):
    for c in checks:
        c()


def _cdiv(a, b):
    return (a + b - 1) // b


def g_quant_act(qr, x, row=True, col=False):
    """qr.quant_act with guarded outputs (checked after the call)."""
    rows, cols = x.shape
    ch = []
    q = s = qT = sT = None
    if row:
        q = guarded_empty((rows, cols), torch.uint8, ch)
        s = guarded_empty((rows, _cdiv(cols, 128)), torch.float32, ch)
    if col:
        qT = guarded_empty((cols, rows), torch.uint8, ch)
        sT = guarded_empty((cols, _cdiv(rows, 128)), torch.float32, ch)
    qr.qr_quant_act_1x128(x, rows, cols, x.stride(0), q, s, qT, sT)
    _run_checks(ch)
    return q, s, qT, sT


def g_quant_w(qr, w, transposed=False):
    n, k = w.shape
    ch = []
    q = guarded_empty((n, k), torch.uint8, ch)
    s = guarded_empty((_cdiv(n, 128), _cdiv(k, 128)), torch.float32, ch)
    qT = sT = None
    if transposed:
        qT = guarded_empty((k, n), torch.uint8, ch)
        sT = guarded_empty((_cdiv(k, 128), _cdiv(n, 128)), torch.float32, ch)
    qr.qr_quant_w_128x128(w, n, k, w.stride(0), q, s, qT, sT)
    _run_checks(ch)
    return q, s, qT, sT


def _od(qr, out_dtype):
    return qr.QR_OUT_BF16 if out_dtype is None else out_dtype


def _g_out_ws(qr, kind, M, N, K, out_dtype, rows, cols, ch):
    if out_dtype is None:
        out_dtype = qr.QR_OUT_BF16
    dt = torch.bfloat16 if out_dtype == qr.QR_OUT_BF16 else torch.float32
    y = guarded_empty((rows, cols), dt, ch)
    nb = qr.qr_gemm_workspace_bytes(kind, M, N, K)
    ws = guarded_empty((nb,), torch.uint8, ch) if nb else None
    return y, ws, nb


def g_gemm_fprop(qr, a, sa, b, sb, out_dtype=None):
    M, K = a.shape
    N = b.shape[0]
    ch = []
    y, ws, nb = _g_out_ws(qr, qr.QR_GEMM_FPROP, M, N, K, out_dtype, M, N, ch)
    qr.qr_gemm_fp8_bsfprop(a, sa, b, sb, M, N, K, y, _od(qr, out_dtype), ws, nb)
    _run_checks(ch)
    return y


def g_gemm_dgrad(qr, dy, sdy, wT, swT, out_dtype=None):
    M, N = dy.shape
    K = wT.shape[0]
    ch = []
    dx, ws, nb = _g_out_ws(qr, qr.QR_GEMM_DGRAD, M, N, K, out_dtype, M, K, ch)
    qr.qr_gemm_fp8_bsdgrad(dy, sdy, wT, swT, M, N, K, dx, _od(qr, out_dtype), ws, nb)
    _run_checks(ch)
    return dx


def g_gemm_wgrad(qr, dyT, sdyT, xT, sxT, out_dtype=None):
    N, M = dyT.shape
    K = xT.shape[0]
    ch = []
    dw, ws, nb = _g_out_ws(qr, qr.QR_GEMM_WGRAD, M, N, K, out_dtype, N, K, ch)
    qr.qr_gemm_fp8_bswgrad(dyT, sdyT, xT, sxT, M, N, K, dw, _od(qr, out_dtype), ws, nb)
    _run_checks(ch)
    return dw
