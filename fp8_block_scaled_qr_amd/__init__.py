"""Python binding of libqr.so, the gfx950 fine-grained FP8 quantize-and-multiply library.

The functions below carry the names of the C entry points declared in include/qr.h and only
marshal arguments: torch tensors on the GPU supply device pointers, torch's current HIP
stream supplies the stream, and every step of the computation runs in the library's HIP
kernels.  There is no CPU fallback: if libqr.so is missing or cannot be loaded, every call
raises.

Each ``qr_*`` function takes preallocated outputs (like the C ABI).  The ``quant_act``,
``quant_w``, ``gemm_*`` and ``uaq_fold`` helpers allocate the outputs with torch and call the
``qr_*`` function.

Before a pointer crosses the boundary, each tensor argument is checked: it must live on a GPU,
have one of the element types the argument takes, have a contiguous last dimension, be
contiguous where the C call takes no leading dimension for it, and span at least the bytes the
call will touch from its first element.  A failed check raises ValueError (TypeError for a
non-tensor) and nothing is launched; the C ABI then validates sizes, alignment and aliasing.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqr.so")

QR_OK = 0
QR_OUT_F32 = 0
QR_OUT_BF16 = 1
QR_GEMM_FPROP, QR_GEMM_DGRAD, QR_GEMM_WGRAD, QR_GEMM_INT8 = 0, 1, 2, 3

# Every entry point include/qr.h declares.
EXPORTS = ("qr_status_string", "qr_abi_version", "qr_quant_act_1x128", "qr_quant_w_128x128",
           "qr_quant_w_128x128_batched", "qr_rmsnorm_quant_1x128", "qr_quant_int8_rowwise",
           "qr_gemm_int8_w8a8", "qr_quant_w_nvfp4", "qr_gemm_w4a16", "qr_gemm_fp8_bsfprop",
           "qr_gemm_fp8_bsdgrad", "qr_gemm_fp8_bswgrad", "qr_gemm_workspace_bytes",
           "qr_uaq_fold", "qr_uaq_fold_quant_w_128x128", "qr_gemm_fp8_bsfprop_noalloc",
           "qr_rmsnorm_quant_dual")
QR_MAX_WEIGHT_BATCH = 4096
QR_NVFP4_WORKSPACE_BYTES = 4096
QR_NOALLOC_SCRATCH_BYTES = 64 << 20


class qr_weight_desc(ctypes.Structure):
    """Mirror of the C struct qr_weight_desc (one weight of a batched quantization)."""
    _fields_ = [("w_bf16", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("ld_w", ctypes.c_int64), ("q", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("qT", ctypes.c_void_p), ("sT", ctypes.c_void_p)]

_lib = None


class QRError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load():
    """Load libqr.so (raises if it is not built or cannot be loaded)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python fp8_block_scaled_qr_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.qr_status_string.argtypes = [I32]
    L.qr_status_string.restype = ctypes.c_char_p
    L.qr_abi_version.argtypes = []
    L.qr_abi_version.restype = I32
    L.qr_quant_act_1x128.argtypes = [P, I64, I64, I64, P, P, P, P, P]
    L.qr_quant_act_1x128.restype = I32
    L.qr_quant_w_128x128.argtypes = [P, I64, I64, I64, P, P, P, P, P]
    L.qr_quant_w_128x128.restype = I32
    L.qr_quant_w_128x128_batched.argtypes = [ctypes.POINTER(qr_weight_desc), I32, P]
    L.qr_quant_w_128x128_batched.restype = I32
    L.qr_rmsnorm_quant_1x128.argtypes = [P, I64, I64, I64, P, ctypes.c_float, P, P, P, P]
    L.qr_rmsnorm_quant_1x128.restype = I32
    L.qr_rmsnorm_quant_dual.argtypes = [P, I64, I64, I64, P, ctypes.c_float, P, P, P, P, P, P, P]
    L.qr_rmsnorm_quant_dual.restype = I32
    L.qr_quant_int8_rowwise.argtypes = [P, I64, I64, I64, P, P, P]
    L.qr_quant_int8_rowwise.restype = I32
    L.qr_gemm_int8_w8a8.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]
    L.qr_gemm_int8_w8a8.restype = I32
    L.qr_quant_w_nvfp4.argtypes = [P, I64, I64, I64, P, P, P, P, SZ, P]
    L.qr_quant_w_nvfp4.restype = I32
    L.qr_gemm_w4a16.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P]
    L.qr_gemm_w4a16.restype = I32
    for name in ("qr_gemm_fp8_bsfprop", "qr_gemm_fp8_bsdgrad", "qr_gemm_fp8_bswgrad"):
        f = getattr(L, name)
        f.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]
        f.restype = I32
    L.qr_gemm_fp8_bsfprop_noalloc.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P]
    L.qr_gemm_fp8_bsfprop_noalloc.restype = I32
    L.qr_gemm_workspace_bytes.argtypes = [I32, I64, I64, I64]
    L.qr_gemm_workspace_bytes.restype = SZ
    L.qr_uaq_fold.argtypes = [P, I64, I64, I64, P, P, P, P]
    L.qr_uaq_fold.restype = I32
    L.qr_uaq_fold_quant_w_128x128.argtypes = [P, I64, I64, I64, P, P, P, P, P, P, P, P]
    L.qr_uaq_fold_quant_w_128x128.restype = I32
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().qr_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load().qr_abi_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_KINDS = {}


def _kinds(kind):
    """Element types an argument of the given kind accepts."""
    if not _KINDS:
        import torch
        _KINDS.update({
            "bf16": (torch.bfloat16, torch.int16, torch.uint16),   # bf16 or its bit patterns
            "f32": (torch.float32,),
            "fp8": (torch.uint8, torch.float8_e4m3fn),               # E4M3 codes
            "u8": (torch.uint8,),
            "i8": (torch.int8,),
            "any": None,
        })
    return _KINDS[kind]


def _arg(t, name, kind, nbytes=0, dense=False):
    """Device pointer of tensor argument t after the checks in the module docstring; None stays
    None (the C ABI decides whether NULL is allowed)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor is on {t.device}; the library takes GPU memory only")
    _check_layout(t, name, kind, nbytes, dense)
    return ctypes.c_void_p(t.data_ptr())


def _check_layout(t, name, kind, nbytes, dense):
    """The element-type, contiguity and extent checks of _arg (independent of the device)."""
    kinds = _kinds(kind)
    if kinds is not None and t.dtype not in kinds:
        raise ValueError(f"{name}: dtype {t.dtype} not accepted (expected one of {kinds})")
    if t.numel() > 0:
        if t.dim() > 0 and t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous (stride 1)")
        if dense and not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous (the call takes no leading dimension)")
        span = 1 + sum((d - 1) * st for d, st in zip(t.shape, t.stride()))
        have = span * t.element_size()
    else:
        have = 0
    if have < nbytes:
        raise ValueError(f"{name}: spans {have} bytes from its first element; the call needs "
                         f"{nbytes}")


def _need(*dims):
    """Product of the sizes, or 0 when any is not positive (the C ABI then launches nothing or
    rejects the shape)."""
    p = 1
    for d in dims:
        if d <= 0:
            return 0
        p *= int(d)
    return p


def _strided(rows, cols, ld, elem):
    """Bytes of a row-major [rows, cols] tensor with leading dimension ld."""
    return 0 if rows <= 0 or cols <= 0 else ((rows - 1) * ld + cols) * elem


def _out_kind(y_dtype):
    return "bf16" if int(y_dtype) == QR_OUT_BF16 else "f32"


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, where):
    if status != QR_OK:
        raise QRError(status, where)


# ------------------------------------------------------------------ C-ABI mirrors

def _cdiv(a, b):
    return (a + b - 1) // b


def qr_quant_act_1x128(x, rows, cols, ld_x, q_row, s_row, q_colT, s_colT, stream=None):
    n, g = _need(rows, cols), _cdiv(cols, 128)
    _check(load().qr_quant_act_1x128(
        _arg(x, "x", "bf16", _strided(rows, cols, ld_x, 2)), rows, cols, ld_x,
        _arg(q_row, "q_row", "fp8", n, True), _arg(s_row, "s_row", "f32", _need(rows, g) * 4, True),
        _arg(q_colT, "q_colT", "fp8", n, True),
        _arg(s_colT, "s_colT", "f32", _need(cols, _cdiv(rows, 128)) * 4, True),
        _stream(stream)), "qr_quant_act_1x128")


def _weight_args(w, n, k, ld_w, q, s, qT, sT, where=""):
    nb = _need(_cdiv(n, 128), _cdiv(k, 128)) * 4 if n > 0 and k > 0 else 0
    return (_arg(w, where + "w", "bf16", _strided(n, k, ld_w, 2)),
            _arg(q, where + "q", "fp8", _need(n, k), True), _arg(s, where + "s", "f32", nb, True),
            _arg(qT, where + "qT", "fp8", _need(n, k), True),
            _arg(sT, where + "sT", "f32", nb, True))


def qr_quant_w_128x128(w, n, k, ld_w, q, s, qT, sT, stream=None):
    pw, pq, ps, pqT, psT = _weight_args(w, n, k, ld_w, q, s, qT, sT)
    _check(load().qr_quant_w_128x128(pw, n, k, ld_w, pq, ps, pqT, psT, _stream(stream)),
           "qr_quant_w_128x128")


def qr_quant_w_128x128_batched(items, stream=None):
    """items: sequence of (w, n, k, ld_w, q, s, qT, sT) as for qr_quant_w_128x128 (qT, sT may
    be None)."""
    arr = (qr_weight_desc * max(1, len(items)))()
    for i, (w, n, k, ld_w, q, s_, qT, sT) in enumerate(items):
        ptrs = _weight_args(w, n, k, ld_w, q, s_, qT, sT, f"items[{i}].")
        vals = [None if p is None else p.value for p in ptrs]
        arr[i] = qr_weight_desc(vals[0], n, k, ld_w, *vals[1:])
    _check(load().qr_quant_w_128x128_batched(arr, len(items), _stream(stream)),
           "qr_quant_w_128x128_batched")


def qr_rmsnorm_quant_1x128(h, rows, cols, ld_h, gain, eps, y, q_row, s_row, stream=None):
    n = _need(rows, cols)
    _check(load().qr_rmsnorm_quant_1x128(
        _arg(h, "h", "bf16", _strided(rows, cols, ld_h, 2)), rows, cols, ld_h,
        _arg(gain, "gain", "f32", _need(cols) * 4, True), float(eps),
        _arg(y, "y", "bf16", n * 2, True), _arg(q_row, "q_row", "fp8", n, True),
        _arg(s_row, "s_row", "f32", _need(rows, _cdiv(cols, 128)) * 4, True), _stream(stream)),
        "qr_rmsnorm_quant_1x128")


def qr_rmsnorm_quant_dual(h, rows, cols, ld_h, gain, eps, inv_rms, y, q_row, s_row, q_colT,
                          s_colT, stream=None):
    n = _need(rows, cols)
    _check(load().qr_rmsnorm_quant_dual(
        _arg(h, "h", "bf16", _strided(rows, cols, ld_h, 2)), rows, cols, ld_h,
        _arg(gain, "gain", "f32", _need(cols) * 4, True), float(eps),
        _arg(inv_rms, "inv_rms", "f32", _need(rows) * 4, True),
        _arg(y, "y", "bf16", n * 2, True), _arg(q_row, "q_row", "fp8", n, True),
        _arg(s_row, "s_row", "f32", _need(rows, _cdiv(cols, 128)) * 4, True),
        _arg(q_colT, "q_colT", "fp8", n, True),
        _arg(s_colT, "s_colT", "f32", _need(cols, _cdiv(rows, 128)) * 4, True),
        _stream(stream)), "qr_rmsnorm_quant_dual")


def qr_quant_int8_rowwise(x, rows, cols, ld_x, q, s, stream=None):
    _check(load().qr_quant_int8_rowwise(
        _arg(x, "x", "bf16", _strided(rows, cols, ld_x, 2)), rows, cols, ld_x,
        _arg(q, "q", "i8", _need(rows, cols), True), _arg(s, "s", "f32", _need(rows) * 4, True),
        _stream(stream)), "qr_quant_int8_rowwise")


def qr_gemm_int8_w8a8(a, sa, b, sb, M, N, K, y, y_dtype, ws=None, ws_bytes=0, stream=None):
    f = load().qr_gemm_int8_w8a8
    esz = 2 if int(y_dtype) == QR_OUT_BF16 else 4
    _check(f(_arg(a, "a", "i8", _need(M, K), True), _arg(sa, "sa", "f32", _need(M) * 4, True),
             _arg(b, "b", "i8", _need(N, K), True), _arg(sb, "sb", "f32", _need(N) * 4, True),
             M, N, K, _arg(y, "y", _out_kind(y_dtype), _need(M, N) * esz, True), int(y_dtype),
             _arg(ws, "ws", "any", int(ws_bytes), True), int(ws_bytes), _stream(stream)),
           "qr_gemm_int8_w8a8")


def qr_quant_w_nvfp4(w, n, k, ld_w, codes, bscale, tscale, ws, ws_bytes, stream=None):
    _check(load().qr_quant_w_nvfp4(
        _arg(w, "w", "bf16", _strided(n, k, ld_w, 2)), n, k, ld_w,
        _arg(codes, "codes", "u8", _need(n, k) // 2, True),
        _arg(bscale, "bscale", "u8", _need(n, k) // 16, True),
        _arg(tscale, "tscale", "f32", 4, True), _arg(ws, "ws", "any", int(ws_bytes), True),
        int(ws_bytes), _stream(stream)), "qr_quant_w_nvfp4")


def qr_gemm_w4a16(x, codes, bscale, tscale, M, N, K, y, y_dtype, stream=None):
    esz = 2 if int(y_dtype) == QR_OUT_BF16 else 4
    _check(load().qr_gemm_w4a16(
        _arg(x, "x", "bf16", _need(M, K) * 2, True),
        _arg(codes, "codes", "u8", _need(N, K) // 2, True),
        _arg(bscale, "bscale", "u8", _need(N, K) // 16, True),
        _arg(tscale, "tscale", "f32", 4 if _need(M, N) else 0, True), M, N, K,
        _arg(y, "y", _out_kind(y_dtype), _need(M, N) * esz, True), int(y_dtype),
        _stream(stream)), "qr_gemm_w4a16")


def qr_gemm_fp8_bsfprop(a, sa, b, sb, M, N, K, y, y_dtype, ws=None, ws_bytes=0, stream=None):
    f = load().qr_gemm_fp8_bsfprop
    esz = 2 if int(y_dtype) == QR_OUT_BF16 else 4
    live = _need(M, N) > 0
    nk = K // 128 if K > 0 else 0
    _check(f(_arg(a, "a", "fp8", _need(M, K) if live else 0, True),
             _arg(sa, "sa", "f32", _need(M, nk) * 4 if live else 0, True),
             _arg(b, "b", "fp8", _need(N, K) if live else 0, True),
             _arg(sb, "sb", "f32", _need(_cdiv(N, 128), nk) * 4 if live else 0, True),
             M, N, K, _arg(y, "y", _out_kind(y_dtype), _need(M, N) * esz, True), int(y_dtype),
             _arg(ws, "ws", "any", int(ws_bytes), True), int(ws_bytes), _stream(stream)),
           "qr_gemm_fp8_bsfprop")


def qr_gemm_fp8_bsfprop_noalloc(a, sa, b, sb, M, N, K, y, y_dtype, stream=None):
    """FProp without a workspace: split partial sums go to the library's device scratch."""
    f = load().qr_gemm_fp8_bsfprop_noalloc
    esz = 2 if int(y_dtype) == QR_OUT_BF16 else 4
    live = _need(M, N) > 0
    nk = K // 128 if K > 0 else 0
    _check(f(_arg(a, "a", "fp8", _need(M, K) if live else 0, True),
             _arg(sa, "sa", "f32", _need(M, nk) * 4 if live else 0, True),
             _arg(b, "b", "fp8", _need(N, K) if live else 0, True),
             _arg(sb, "sb", "f32", _need(_cdiv(N, 128), nk) * 4 if live else 0, True),
             M, N, K, _arg(y, "y", _out_kind(y_dtype), _need(M, N) * esz, True), int(y_dtype),
             _stream(stream)), "qr_gemm_fp8_bsfprop_noalloc")


def qr_gemm_fp8_bsdgrad(dy, sdy, wT, swT, M, N, K, dx, dx_dtype, ws=None, ws_bytes=0,
                        stream=None):
    """dX [M, K] = dY [M, N] . W [N, K], with the transposed weight copy wT [K, N]."""
    f = load().qr_gemm_fp8_bsdgrad
    esz = 2 if int(dx_dtype) == QR_OUT_BF16 else 4
    live = _need(M, K) > 0
    nn = N // 128 if N > 0 else 0
    _check(f(_arg(dy, "dy", "fp8", _need(M, N) if live else 0, True),
             _arg(sdy, "sdy", "f32", _need(M, nn) * 4 if live else 0, True),
             _arg(wT, "wT", "fp8", _need(K, N) if live else 0, True),
             _arg(swT, "swT", "f32", _need(_cdiv(K, 128), nn) * 4 if live else 0, True),
             M, N, K, _arg(dx, "dx", _out_kind(dx_dtype), _need(M, K) * esz, True),
             int(dx_dtype), _arg(ws, "ws", "any", int(ws_bytes), True), int(ws_bytes),
             _stream(stream)), "qr_gemm_fp8_bsdgrad")


def qr_gemm_fp8_bswgrad(dyT, sdyT, xT, sxT, M, N, K, dw, dw_dtype, ws=None, ws_bytes=0,
                        stream=None):
    """dW [N, K] = dY^T . X over M tokens, with dY^T [N, M] and X^T [K, M] (128x1 groups)."""
    f = load().qr_gemm_fp8_bswgrad
    esz = 2 if int(dw_dtype) == QR_OUT_BF16 else 4
    live = _need(N, K) > 0
    nm = M // 128 if M > 0 else 0
    _check(f(_arg(dyT, "dyT", "fp8", _need(N, M) if live else 0, True),
             _arg(sdyT, "sdyT", "f32", _need(N, nm) * 4 if live else 0, True),
             _arg(xT, "xT", "fp8", _need(K, M) if live else 0, True),
             _arg(sxT, "sxT", "f32", _need(K, nm) * 4 if live else 0, True),
             M, N, K, _arg(dw, "dw", _out_kind(dw_dtype), _need(N, K) * esz, True),
             int(dw_dtype), _arg(ws, "ws", "any", int(ws_bytes), True), int(ws_bytes),
             _stream(stream)), "qr_gemm_fp8_bswgrad")


def qr_gemm_workspace_bytes(kind, M, N, K) -> int:
    return int(load().qr_gemm_workspace_bytes(int(kind), M, N, K))


def _same_ptr(a, b):
    return a is not None and b is not None and a.data_ptr() == b.data_ptr()


def qr_uaq_fold(w, n, k, ld_w, s, w_out, gain=None, stream=None):
    ld_out = ld_w if _same_ptr(w_out, w) else k
    _check(load().qr_uaq_fold(
        _arg(w, "w", "bf16", _strided(n, k, ld_w, 2)), n, k, ld_w,
        _arg(s, "s", "f32", _need(n, k) and k * 4, True),
        _arg(w_out, "w_out", "bf16", _strided(n, k, ld_out, 2)),
        _arg(gain, "gain", "f32", _need(n, k) and k * 4, True), _stream(stream)), "qr_uaq_fold")


def qr_uaq_fold_quant_w_128x128(w, n, k, ld_w, s, w_out, gain, q, sq, qT=None, sqT=None,
                                stream=None):
    ld_out = ld_w if _same_ptr(w_out, w) else k
    pw, pq, ps, pqT, psT = _weight_args(w, n, k, ld_w, q, sq, qT, sqT)
    _check(load().qr_uaq_fold_quant_w_128x128(
        pw, n, k, ld_w, _arg(s, "s", "f32", _need(n, k) and k * 4, True),
        _arg(w_out, "w_out", "bf16", _strided(n, k, ld_out, 2)),
        _arg(gain, "gain", "f32", _need(n, k) and k * 4, True), pq, ps, pqT, psT,
        _stream(stream)), "qr_uaq_fold_quant_w_128x128")


# ------------------------------------------------------------------ allocating helpers


def quant_act(x, row=True, col=False, stream=None):
    """x: bf16 [rows, cols] on the GPU.  Returns (q_row, s_row, q_colT, s_colT), with None for
    the pair not requested."""
    import torch
    rows, cols = x.shape
    dev = x.device
    q_row = s_row = q_colT = s_colT = None
    if row:
        q_row = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s_row = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.float32, device=dev)
    if col:
        q_colT = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        s_colT = torch.empty((cols, _cdiv(rows, 128)), dtype=torch.float32, device=dev)
    qr_quant_act_1x128(x, rows, cols, x.stride(0), q_row, s_row, q_colT, s_colT, stream)
    return q_row, s_row, q_colT, s_colT


def quant_w(w, transposed=False, stream=None):
    """w: bf16 [n, k] on the GPU.  Returns (q, s, qT, sT) (qT, sT None unless transposed)."""
    import torch
    n, k = w.shape
    dev = w.device
    q = torch.empty((n, k), dtype=torch.uint8, device=dev)
    s = torch.empty((_cdiv(n, 128), _cdiv(k, 128)), dtype=torch.float32, device=dev)
    qT = sT = None
    if transposed:
        qT = torch.empty((k, n), dtype=torch.uint8, device=dev)
        sT = torch.empty((_cdiv(k, 128), _cdiv(n, 128)), dtype=torch.float32, device=dev)
    qr_quant_w_128x128(w, n, k, w.stride(0), q, s, qT, sT, stream)
    return q, s, qT, sT



def quant_w_batched(ws, transposed=False, stream=None):
    """ws: list of bf16 [n, k] weights on the GPU, quantized in one call.  Returns a list of
    (q, s, qT, sT) per weight; transposed is a bool or a list of bools."""
    import torch
    flags = transposed if isinstance(transposed, (list, tuple)) else [transposed] * len(ws)
    outs, items = [], []
    for w, t in zip(ws, flags):
        n, k = w.shape
        dev = w.device
        q = torch.empty((n, k), dtype=torch.uint8, device=dev)
        s = torch.empty((_cdiv(n, 128), _cdiv(k, 128)), dtype=torch.float32, device=dev)
        qT = sT = None
        if t:
            qT = torch.empty((k, n), dtype=torch.uint8, device=dev)
            sT = torch.empty((_cdiv(k, 128), _cdiv(n, 128)), dtype=torch.float32, device=dev)
        outs.append((q, s, qT, sT))
        items.append((w, n, k, w.stride(0), q, s, qT, sT))
    qr_quant_w_128x128_batched(items, stream)
    return outs

def rmsnorm_quant(h, gain, eps=1e-6, want_y=True, stream=None):
    """h: bf16 [rows, cols] on the GPU, gain fp32 [cols].  Returns (y or None, q, s)."""
    import torch
    rows, cols = h.shape
    dev = h.device
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev) if want_y else None
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    s = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.float32, device=dev)
    qr_rmsnorm_quant_1x128(h, rows, cols, h.stride(0), gain, eps, y, q, s, stream)
    return y, q, s


def rmsnorm_quant_dual(h, gain, eps=1e-6, row=True, col=True, want_y=False, stream=None):
    """h: bf16 [rows, cols] on the GPU, gain fp32 [cols].  Returns (inv_rms, y or None, q_row,
    s_row, q_colT, s_colT), with None for the pair not requested."""
    import torch
    rows, cols = h.shape
    dev = h.device
    inv = torch.empty(rows, dtype=torch.float32, device=dev)
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev) if want_y else None
    q_row = s_row = q_colT = s_colT = None
    if row:
        q_row = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s_row = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.float32, device=dev)
    if col:
        q_colT = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        s_colT = torch.empty((cols, _cdiv(rows, 128)), dtype=torch.float32, device=dev)
    qr_rmsnorm_quant_dual(h, rows, cols, h.stride(0), gain, eps, inv, y, q_row, s_row, q_colT,
                          s_colT, stream)
    return inv, y, q_row, s_row, q_colT, s_colT


def quant_int8(x, stream=None):
    """x: bf16 [rows, cols] on the GPU -> (q int8 [rows, cols], s fp32 [rows])."""
    import torch
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    qr_quant_int8_rowwise(x, rows, cols, x.stride(0), q, s, stream)
    return q, s


def gemm_int8(a, sa, b, sb, out_dtype=QR_OUT_BF16, stream=None):
    """a int8 [M, K] with sa [M], b int8 [N, K] with sb [N] -> y [M, N]."""
    M, K = a.shape
    N = b.shape[0]
    y = _out(M, N, out_dtype, a.device)
    ws, nb = _workspace(QR_GEMM_INT8, M, N, K, a.device)
    qr_gemm_int8_w8a8(a, sa, b, sb, M, N, K, y, out_dtype, ws, nb, stream)
    return y


def quant_nvfp4(w, stream=None):
    """w: bf16 [n, k] on the GPU -> (codes u8 [n, k/2], block scales u8 [n, k/16], tensor scale
    fp32 [1])."""
    import torch
    n, k = w.shape
    dev = w.device
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    bs = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
    t = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(QR_NVFP4_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    qr_quant_w_nvfp4(w, n, k, w.stride(0), codes, bs, t, ws, QR_NVFP4_WORKSPACE_BYTES, stream)
    return codes, bs, t


def gemm_w4a16(x, codes, bscale, tscale, out_dtype=QR_OUT_BF16, stream=None):
    """x bf16 [M, K]; the 4-bit weight [N, K] -> y [M, N]."""
    M, K = x.shape
    N = codes.shape[0]
    y = _out(M, N, out_dtype, x.device)
    qr_gemm_w4a16(x, codes, bscale, tscale, M, N, K, y, out_dtype, stream)
    return y


def _workspace(kind, M, N, K, device):
    import torch
    nb = qr_gemm_workspace_bytes(kind, M, N, K)
    return (torch.empty(nb, dtype=torch.uint8, device=device) if nb else None), nb


def _out(M, N, out_dtype, device):
    import torch
    return torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == QR_OUT_BF16 else torch.float32,
                       device=device)


def gemm_fprop(a, sa, b, sb, out_dtype=QR_OUT_BF16, stream=None):
    M, K = a.shape
    N = b.shape[0]
    y = _out(M, N, out_dtype, a.device)
    ws, nb = _workspace(QR_GEMM_FPROP, M, N, K, a.device)
    qr_gemm_fp8_bsfprop(a, sa, b, sb, M, N, K, y, out_dtype, ws, nb, stream)
    return y


def gemm_dgrad(dy, sdy, wT, swT, out_dtype=QR_OUT_BF16, stream=None):
    M, N = dy.shape
    K = wT.shape[0]
    dx = _out(M, K, out_dtype, dy.device)
    ws, nb = _workspace(QR_GEMM_DGRAD, M, N, K, dy.device)
    qr_gemm_fp8_bsdgrad(dy, sdy, wT, swT, M, N, K, dx, out_dtype, ws, nb, stream)
    return dx


def gemm_wgrad(dyT, sdyT, xT, sxT, out_dtype=QR_OUT_BF16, stream=None):
    N, M = dyT.shape
    K = xT.shape[0]
    dw = _out(N, K, out_dtype, dyT.device)
    ws, nb = _workspace(QR_GEMM_WGRAD, M, N, K, dyT.device)
    qr_gemm_fp8_bswgrad(dyT, sdyT, xT, sxT, M, N, K, dw, out_dtype, ws, nb, stream)
    return dw


def uaq_fold(w, s, gain=None, inplace=False, stream=None):
    """Returns the folded weight (bf16); gain (fp32, may be None) is updated in place."""
    import torch
    n, k = w.shape
    out = w if inplace else torch.empty((n, k), dtype=w.dtype, device=w.device)
    qr_uaq_fold(w, n, k, w.stride(0), s, out, gain, stream)
    return out


def uaq_fold_quant_w(w, s, gain=None, transposed=False, inplace=False, stream=None):
    """The fold and the 128x128 quantization in one pass.  Returns (w_folded, q, sq, qT, sqT)
    (qT, sqT None unless transposed); gain (fp32, may be None) is updated in place."""
    import torch
    n, k = w.shape
    dev = w.device
    out = w if inplace else torch.empty((n, k), dtype=w.dtype, device=dev)
    q = torch.empty((n, k), dtype=torch.uint8, device=dev)
    sq = torch.empty((_cdiv(n, 128), _cdiv(k, 128)), dtype=torch.float32, device=dev)
    qT = sqT = None
    if transposed:
        qT = torch.empty((k, n), dtype=torch.uint8, device=dev)
        sqT = torch.empty((_cdiv(k, 128), _cdiv(n, 128)), dtype=torch.float32, device=dev)
    qr_uaq_fold_quant_w_128x128(w, n, k, w.stride(0), s, out, gain, q, sq, qT, sqT, stream)
    return out, q, sq, qT, sqT
