"""The C ABI without a GPU: the library loads, exports every entry point the header declares,
and rejects invalid arguments with the documented status before any HIP call.  Only argument
combinations that fail validation (or have a zero size, which launches nothing) are used, so
no kernel is ever launched here; the pointers are fake and never dereferenced."""
import ctypes
import os
import re
import subprocess

import pytest

import fp8_block_scaled_qr_amd as qr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, ALIGN, ALIAS, WORKSPACE, LAUNCH, ARG, SCRATCH = range(9)

A = 1 << 40          # fake, 16-byte aligned device addresses far apart
B = 2 << 40
C = 3 << 40
D = 4 << 40
E = 5 << 40


def header_functions():
    text = open(os.path.join(ROOT, "include", "qr.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qr_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    return qr.load()


def test_exports_match_header(L):
    declared = header_functions()
    assert len(declared) == 18, declared
    out = subprocess.run(["nm", "-D", "--defined-only", qr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("qr_"))
    assert exported == declared
    assert sorted(qr.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name)


def test_status_strings_and_version(L):
    assert qr.abi_version() == 4
    for st in range(9):
        assert qr.status_string(st)
    assert "unknown" in qr.status_string(99)


def act(L, x, rows, cols, ld, q, s, qT, sT):
    return L.qr_quant_act_1x128(x, rows, cols, ld, q, s, qT, sT, None)


def test_quant_act_validation(L):
    assert act(L, A, -1, 128, 128, B, C, None, None) == SHAPE
    assert act(L, A, 4, 100, 104, B, C, None, None) == SHAPE          # cols % 8
    assert act(L, A, 4, 128, 100, B, C, None, None) == SHAPE          # ld < cols
    assert act(L, A, 4, 128, 132, B, C, None, None) == SHAPE          # ld % 8
    assert act(L, A, 12, 128, 128, None, None, B, C) == SHAPE         # column pass: rows % 8
    assert act(L, A, 4, 128, 128, None, None, None, None) == NULL     # no output
    assert act(L, A, 4, 128, 128, B, None, None, None) == NULL        # half a pair
    assert act(L, None, 4, 128, 128, B, C, None, None) == NULL
    assert act(L, A + 2, 8, 128, 128, B, C, None, None) == ALIGN
    assert act(L, A, 8, 128, 128, B + 8, C, None, None) == ALIGN
    assert act(L, A, 8, 128, 128, B, C + 2, None, None) == ALIGN
    assert act(L, A, 8, 128, 128, A + 16, C, None, None) == ALIAS     # codes inside x
    assert act(L, A, 8, 128, 128, B, B + 512, None, None) == ALIAS    # scales inside codes
    assert act(L, A, 8, 128, 128, B, C, B + 512, D) == ALIAS          # colT over row codes
    assert act(L, A, 0, 128, 128, B, C, None, None) == OK             # empty: nothing launched
    assert act(L, A, 8, 0, 0, B, C, D, E) == OK
    assert act(L, A, 128 * 65536, 8, 8, B, C, None, None) == SHAPE   # row tiles beyond grid


def test_quant_w_validation(L):
    f = L.qr_quant_w_128x128
    assert f(A, 128, 128, 128, None, C, None, None, None) == NULL
    assert f(A, 128, 128, 128, B, C, D, None, None) == NULL          # half of the T pair
    assert f(A, 100, 128, 128, B, C, None, None, None) == SHAPE       # n % 8
    assert f(A, 128, 124, 128, B, C, None, None, None) == SHAPE       # k % 8
    assert f(A + 8, 128, 128, 128, B, C, None, None, None) == ALIGN
    assert f(A, 128, 128, 128, B, A, None, None, None) == ALIAS
    assert f(A, 128, 128, 128, B, C, B + 64, D, None) == ALIAS
    assert f(A, 0, 128, 128, B, C, None, None, None) == OK


def test_rmsnorm_quant_validation(L):
    f = L.qr_rmsnorm_quant_1x128
    assert f(A, -1, 128, 128, B, 1e-6, None, C, D, None) == SHAPE
    assert f(A, 4, 100, 104, B, 1e-6, None, C, D, None) == SHAPE         # cols % 8
    assert f(A, 4, 128, 120, B, 1e-6, None, C, D, None) == SHAPE         # ld < cols
    assert f(A, 4, 128, 128, B, -1.0, None, C, D, None) == ARG           # eps < 0
    assert f(A, 4, 128, 128, B, float("nan"), None, C, D, None) == ARG
    assert f(A, 4, 128, 128, None, 1e-6, None, C, D, None) == NULL       # gain required
    assert f(A, 4, 128, 128, B, 1e-6, None, None, D, None) == NULL
    assert f(A + 2, 4, 128, 128, B, 1e-6, None, C, D, None) == ALIGN
    assert f(A, 4, 128, 128, B + 4, 1e-6, None, C, D, None) == ALIGN     # gain 16-byte
    assert f(A, 4, 128, 128, B, 1e-6, E + 8, C, D, None) == ALIGN        # y 16-byte
    assert f(A, 4, 128, 128, B, 1e-6, None, A + 64, D, None) == ALIAS    # codes over h
    assert f(A, 4, 128, 128, B, 1e-6, C + 256, C, D, None) == ALIAS      # y over codes
    assert f(A, 4, 128, 128, B, 1e-6, None, C, B + 16, None) == ALIAS    # scales over gain
    assert f(A, 0, 128, 128, B, 1e-6, None, C, D, None) == OK


def test_int8_validation(L):
    f = L.qr_quant_int8_rowwise
    assert f(A, -1, 128, 128, B, C, None) == SHAPE
    assert f(A, 4, 100, 104, B, C, None) == SHAPE                        # cols % 8
    assert f(A, 4, 128, 120, B, C, None) == SHAPE                        # ld < cols
    assert f(A, 4, 128, 128, None, C, None) == NULL
    assert f(A + 2, 4, 128, 128, B, C, None) == ALIGN
    assert f(A, 4, 128, 128, B + 8, C, None) == ALIGN
    assert f(A, 4, 128, 128, A + 16, C, None) == ALIAS                   # codes over x
    assert f(A, 4, 128, 128, B, B + 256, None) == ALIAS                  # scales over codes
    assert f(A, 0, 128, 128, B, C, None) == OK
    g = L.qr_gemm_int8_w8a8
    assert g(A, B, C, D, 64, 64, 100, E, 1, None, 0, None) == SHAPE               # K % 128
    assert g(A, B, C, D, 64, 64, 131072 + 128, E, 1, None, 0, None) == SHAPE      # int32 range
    assert g(A, B, C, D, 64, 64, 128, E, 7, None, 0, None) == ARG                 # output dtype
    assert g(None, B, C, D, 64, 64, 128, E, 1, None, 0, None) == NULL
    assert g(A, B, C + 4, D, 64, 64, 128, E, 1, None, 0, None) == ALIGN
    assert g(A, B, C, D, 64, 64, 128, A + 1024, 1, None, 0, None) == ALIAS        # y over a
    assert g(A, B, C, D, 0, 64, 128, E, 1, None, 0, None) == OK
    # a split product (few 256x256 tiles) needs the workspace for its int32 partials
    W, nb = 6 << 40, qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, 256, 5120, 27648)
    assert g(A, B, C, D, 256, 5120, 27648, E, 1, None, 0, None) == WORKSPACE
    assert g(A, B, C, D, 256, 5120, 27648, E, 1, W, nb - 1, None) == WORKSPACE
    assert g(A, B, C, D, 256, 5120, 27648, E, 1, W + 8, nb, None) == ALIGN
    assert g(A, B, C, D, 256, 5120, 27648, E, 1, C + 4096, nb, None) == ALIAS     # ws over b
    assert g(A, B, C, D, 256, 5120, 27648, E, 1, E + 4096, nb, None) == ALIAS     # ws over y


def test_fold_quant_w_validation(L):
    f = L.qr_uaq_fold_quant_w_128x128
    F = 6 << 40
    # (w, n, k, ld_w, s, w_out, gain, q, sq, qT, sqT, stream)
    assert f(A, 128, 100, 104, B, C, None, D, E, None, None, None) == SHAPE   # k % 8
    assert f(A, 100, 128, 128, B, C, None, D, E, None, None, None) == SHAPE   # n % 8
    assert f(A, 128, 128, 120, B, C, None, D, E, None, None, None) == SHAPE   # ld < k
    assert f(A, 128, 128, 128, B, C, None, None, E, None, None, None) == NULL  # codes
    assert f(A, 128, 128, 128, B, C, None, D, E, F, None, None) == NULL        # qT without sT
    assert f(A, 128, 128, 128, None, C, None, D, E, None, None, None) == NULL  # s
    assert f(A, 128, 128, 128, B, None, None, D, E, None, None, None) == NULL  # w_out
    assert f(A, 128, 128, 128, B + 4, C, None, D, E, None, None, None) == ALIGN   # s 16-byte
    assert f(A, 128, 128, 128, B, C + 8, None, D, E, None, None, None) == ALIGN   # w_out
    assert f(A, 128, 128, 128, B, C, E + 2, D, E + 1024, None, None, None) == ALIGN  # gain
    assert f(A, 128, 128, 128, B, A + 256, None, D, E, None, None, None) == ALIAS  # w_out over w
    assert f(A, 128, 128, 128, B, C, B + 16, D, E, None, None, None) == ALIAS     # gain over s
    assert f(A, 128, 128, 128, B, C, None, C + 64, E, None, None, None) == ALIAS  # q over w_out
    assert f(A, 128, 128, 128, B, C, None, D, E, D + 64, E + 1024, None) == ALIAS  # qT over q
    assert f(A, 0, 128, 128, B, C, None, D, E, None, None, None) == OK


def test_fp4_validation(L):
    f = L.qr_quant_w_nvfp4
    WS = qr.QR_NVFP4_WORKSPACE_BYTES
    assert f(A, 128, 48, 48, B, C, D, E, WS, None) == SHAPE             # k % 32
    assert f(A, 128, 128, 120, B, C, D, E, WS, None) == SHAPE           # ld < k
    assert f(A, 128, 128, 128, None, C, D, E, WS, None) == NULL
    assert f(A, 128, 128, 128, B, C, D, None, WS, None) == NULL         # workspace required
    assert f(A, 128, 128, 128, B, C, D, E, WS - 4, None) == WORKSPACE
    assert f(A + 2, 128, 128, 128, B, C, D, E, WS, None) == ALIGN
    assert f(A, 128, 128, 128, A + 64, C, D, E, WS, None) == ALIAS      # codes over w
    assert f(A, 128, 128, 128, B, C, D, C + 4, WS, None) == ALIAS       # workspace over scales
    assert f(A, 0, 128, 128, B, C, D, E, WS, None) == OK
    g = L.qr_gemm_w4a16
    assert g(A, B, C, D, 64, 64, 96, E, 1, None) == SHAPE               # K % 128
    assert g(A, B, C, D, 64, 64, 128, E, 5, None) == ARG
    assert g(A, None, C, D, 64, 64, 128, E, 1, None) == NULL
    assert g(A, B, C + 1, D, 64, 64, 128, E, 1, None) == ALIGN          # bscale 2-byte
    assert g(A, B, C, D, 64, 64, 128, B + 64, 1, None) == ALIAS         # y over codes
    assert g(A, B, C, D, 64, 0, 128, E, 1, None) == OK


def batch(L, descs):
    arr = (qr.qr_weight_desc * max(1, len(descs)))(*[qr.qr_weight_desc(*d) for d in descs])
    return L.qr_quant_w_128x128_batched(arr, len(descs), None)


def test_quant_w_batched_validation(L):
    f = L.qr_quant_w_128x128_batched
    assert f(None, 0, None) == OK                                     # nothing to do
    assert f(None, 1, None) == NULL
    arr = (qr.qr_weight_desc * 1)()
    assert f(arr, -1, None) == SHAPE
    assert f(arr, qr.QR_MAX_WEIGHT_BATCH + 1, None) == SHAPE
    M = 1 << 20                                                       # 1 MiB apart
    good0 = (A, 128, 128, 128, B, C, None, None)
    good1 = (A + M, 256, 128, 128, B + M, C + M, D, E)
    # each descriptor is checked like qr_quant_w_128x128
    assert batch(L, [good0, (A + M, 100, 128, 128, B + M, C + M, None, None)]) == SHAPE
    assert batch(L, [good0, (A + M, 128, 128, 128, None, C + M, None, None)]) == NULL
    assert batch(L, [good0, (A + M, 128, 128, 128, B + M, C + M, D, None)]) == NULL
    assert batch(L, [(A + 8, 128, 128, 128, B, C, None, None), good1]) == ALIGN
    # aliasing across descriptors: an output over another weight's input or output
    assert batch(L, [good0, (A + M, 128, 128, 128, A + 64, C + M, None, None)]) == ALIAS
    assert batch(L, [good0, (A + M, 128, 128, 128, B + M, B + 64, None, None)]) == ALIAS
    assert batch(L, [good0, (A + M, 256, 128, 128, B + M, C + M, B + 128, E)]) == ALIAS
    assert batch(L, [good0, (A + M, 128, 128, 128, B + M, C, None, None)]) == ALIAS
    assert batch(L, [good1, (A, 128, 128, 128, B, C, None, None),
                     (A + 2 * M, 8, 8, 8, A + M + 32, C + 2 * M, None, None)]) == ALIAS
    # empty weights are skipped (nothing launched)
    assert batch(L, [(A, 0, 128, 128, B, C, None, None), (A, 128, 0, 0, B, C, D, E)]) == OK


def gemm(L, name, a, sa, b, sb, M, N, K, y, dt, ws, wsb):
    return getattr(L, name)(a, sa, b, sb, M, N, K, y, dt, ws, wsb, None)


@pytest.mark.parametrize("name", ["qr_gemm_fp8_bsfprop", "qr_gemm_fp8_bsdgrad",
                                  "qr_gemm_fp8_bswgrad"])
def test_gemm_validation(L, name):
    # the contraction size is K for FProp, N for DGrad, M for WGrad
    contraction = {"qr_gemm_fp8_bsfprop": 2, "qr_gemm_fp8_bsdgrad": 1, "qr_gemm_fp8_bswgrad": 0}[name]
    kind = {"qr_gemm_fp8_bsfprop": 0, "qr_gemm_fp8_bsdgrad": 1, "qr_gemm_fp8_bswgrad": 2}[name]
    # shapes whose plans split K, so that a workspace is needed: 128 rows (64x64 decode tiles,
    # 4 and 2 splits) for FProp and DGrad, dW 512x1024 over 4096 tokens (64x64 tiles, 2 splits)
    # for WGrad
    dims = [4096, 512, 1024] if kind == 2 else [128, 2048, 4096]
    bad = list(dims)
    bad[contraction] = 200
    assert gemm(L, name, A, B, C, D, *bad, E, 1, None, 0) == SHAPE
    assert gemm(L, name, A, B, C, D, -1, 2048, 2048, E, 1, None, 0) == SHAPE
    assert gemm(L, name, A, B, C, D, *dims, E, 7, None, 0) == ARG
    assert gemm(L, name, None, B, C, D, *dims, E, 1, None, 0) == NULL
    assert gemm(L, name, A, B, C, D, *dims, None, 1, None, 0) == NULL
    assert gemm(L, name, A + 4, B, C, D, *dims, E, 1, None, 0) == ALIGN
    assert gemm(L, name, A, B + 2, C, D, *dims, E, 1, None, 0) == ALIGN
    ws, wsb = 6 << 40, qr.qr_gemm_workspace_bytes(kind, *dims)
    assert wsb > 0
    assert gemm(L, name, A, B, C, D, *dims, E, 1, None, 0) == WORKSPACE
    assert gemm(L, name, A, B, C, D, *dims, A + 64, 1, ws, wsb) == ALIAS    # output over A
    assert gemm(L, name, A, B, C, D, *dims, C, 0, ws, wsb) == ALIAS         # output over B
    z = list(dims)
    z[[0, 1, 2][contraction - 1]] = 0                                         # an output dim 0
    assert gemm(L, name, A, B, C, D, *z, E, 1, None, 0) == OK


def test_gemm_workspace(L):
    # mid-size M (65..256) splits K over a few tiles and needs a workspace; decode batches up
    # to 64 rows stream a wide weight without a split, and split K over a narrow one; large
    # shapes need none
    nb = qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 200, 14336, 4096)
    assert nb > 0 and nb % (200 * 14336 * 4) == 0
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 64, 14336, 4096) == 0
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 64, 4096, 4096) == 4 * 64 * 4096 * 4
    # decode batches: 64-wide tiles split K only while they give at most 128 workgroups (8192
    # columns: 128 tiles x 2 splits; one more tile column: no split); 128-wide tiles (more than
    # 256 tiles of 64) never split
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 64, 8192, 4096) == 2 * 64 * 8192 * 4
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 64, 8256, 4096) == 0
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 64, 28672, 4096) == 0
    # 65..256 rows: 256x128 tiles where 256x256 ones would split K so far that the partials
    # outweigh the weight (QKV of the 32B layer: 56 tiles x 4 splits), 256x256 tiles otherwise
    # (its down projection: 20 tiles x 12 splits)
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 256, 7168, 5120) == 4 * 256 * 7168 * 4
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 256, 5120, 27648) == 12 * 256 * 5120 * 4
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 8192, 4096, 4096) == 0
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, 200, 14336, 100) == 0    # invalid K
    assert qr.qr_gemm_workspace_bytes(9, 200, 14336, 4096) == 0
    assert gemm(L, "qr_gemm_fp8_bsfprop", A, B, C, D, 200, 14336, 4096, E, 1, None, 0) == WORKSPACE
    assert gemm(L, "qr_gemm_fp8_bsfprop", A, B, C, D, 200, 14336, 4096, E, 1, 6 << 40, nb - 1) == WORKSPACE
    assert gemm(L, "qr_gemm_fp8_bsfprop", A, B, C, D, 200, 14336, 4096, E, 1, A, nb) == ALIAS
    # DGrad / WGrad sizes are passed as given to their entry points
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_DGRAD, 200, 4096, 14336) > 0
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_WGRAD, 8192, 4096, 4096) == 0
    # INT8: int32 partials; 256 rows against a 5120-wide weight give 20 tiles x 12 splits, a
    # 64-row batch against a 4096-wide one 64 tiles of 64x64 x 4 splits
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, 256, 5120, 27648) == 12 * 256 * 5120 * 4
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, 64, 4096, 14336) == 4 * 64 * 4096 * 4
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, 64, 14336, 4096) == 0
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, 8192, 4096, 4096) == 0
    assert qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, 64, 64, 131072 + 128) == 0  # invalid K


def test_uaq_validation(L):
    f = L.qr_uaq_fold
    assert f(A, 4, 100, 104, B, C, None, None) == SHAPE                # k % 8
    assert f(A, 4, 128, 120, B, C, None, None) == SHAPE                # ld < k
    assert f(None, 4, 128, 128, B, C, None, None) == NULL
    assert f(A, 4, 128, 128, None, C, None, None) == NULL
    assert f(A, 4, 128, 128, B + 4, C, None, None) == ALIGN            # s is read as float4
    assert f(A, 4, 128, 128, B, A + 256, None, None) == ALIAS          # partial overlap
    assert f(A, 4, 128, 128, B, C, B, None) == ALIAS                   # gain over s
    assert f(A, 0, 128, 128, B, C, D, None) == OK


def test_binding_rejects_host_tensors():
    """Every binding entry point raises before the call when handed host memory (a host
    pointer in a kernel would fault the device)."""
    import torch
    x = torch.zeros((8, 128), dtype=torch.bfloat16)
    codes = torch.zeros((8, 128), dtype=torch.uint8)
    sc = torch.zeros((8, 1), dtype=torch.float32)
    y = torch.zeros((8, 128), dtype=torch.float32)
    calls = [
        lambda: qr.qr_quant_act_1x128(x, 8, 128, 128, codes, sc, None, None),
        lambda: qr.qr_quant_w_128x128(x, 8, 128, 128, codes, sc, None, None),
        lambda: qr.qr_quant_w_128x128_batched([(x, 8, 128, 128, codes, sc, None, None)]),
        lambda: qr.qr_rmsnorm_quant_1x128(x, 8, 128, 128, sc, 1e-6, None, codes, sc),
        lambda: qr.qr_quant_int8_rowwise(x, 8, 128, 128, codes.view(torch.int8), sc),
        lambda: qr.qr_gemm_fp8_bsfprop(codes, sc, codes, sc, 8, 128, 128, y, qr.QR_OUT_F32),
        lambda: qr.qr_gemm_fp8_bsdgrad(codes, sc, codes, sc, 8, 128, 128, y, qr.QR_OUT_F32),
        lambda: qr.qr_gemm_fp8_bswgrad(codes, sc, codes, sc, 128, 8, 8, y, qr.QR_OUT_F32),
        lambda: qr.qr_uaq_fold(x, 8, 128, 128, sc, x),
        lambda: qr.quant_act(x), lambda: qr.quant_w(x), lambda: qr.gemm_fprop(codes, sc, codes, sc),
    ]
    for c in calls:
        with pytest.raises(ValueError, match="GPU memory only"):
            c()
    with pytest.raises(TypeError):
        qr.qr_quant_act_1x128(123, 8, 128, 128, None, None, None, None)


def test_binding_layout_checks():
    """The dtype, contiguity and extent checks the binding applies to every tensor argument."""
    import torch
    w = torch.zeros((256, 640), dtype=torch.bfloat16)
    qr._check_layout(w[:, 64:448], "w", "bf16", (255 * 640 + 384) * 2, False)   # strided rows ok
    with pytest.raises(ValueError, match="last dimension"):
        qr._check_layout(w[:, ::2], "w", "bf16", 2, False)                       # column stride 2
    with pytest.raises(ValueError, match="contiguous"):
        qr._check_layout(w[:, :128], "q", "bf16", 2, True)                        # dense required
    with pytest.raises(ValueError, match="spans"):
        qr._check_layout(w[:2], "w", "bf16", 3 * 640 * 2, False)                  # too short
    with pytest.raises(ValueError, match="dtype"):
        qr._check_layout(w.float(), "x", "bf16", 0, False)
    with pytest.raises(ValueError, match="dtype"):
        qr._check_layout(torch.zeros(4, dtype=torch.int8), "q", "fp8", 0, True)
    qr._check_layout(torch.zeros(4, dtype=torch.int16), "x", "bf16", 8, True)     # bit patterns
    qr._check_layout(torch.zeros(0, dtype=torch.float32), "ws", "any", 0, True)   # empty, none needed
    with pytest.raises(ValueError, match="spans"):
        qr._check_layout(torch.zeros(0, dtype=torch.uint8), "ws", "any", 16, True)


def test_gemm_noalloc_validation(L):
    """The allocation-free FProp validates like qr_gemm_fp8_bsfprop (no workspace argument)."""
    f = L.qr_gemm_fp8_bsfprop_noalloc
    assert f(A, B, C, D, 8, 128, 100, E, 1, None) == SHAPE           # K % 128
    assert f(A, B, C, D, -1, 128, 128, E, 1, None) == SHAPE
    assert f(A, B, C, D, 8, 128, 128, E, 2, None) == ARG              # output dtype
    assert f(None, B, C, D, 8, 128, 128, E, 1, None) == NULL
    assert f(A, B, C, D, 8, 128, 128, None, 1, None) == NULL
    assert f(A + 4, B, C, D, 8, 128, 128, E, 1, None) == ALIGN
    assert f(A, B, C, D, 8, 128, 128, A + 512, 1, None) == ALIAS      # y inside a
    assert f(A, B, C, D, 0, 128, 128, E, 1, None) == OK               # empty: nothing launched
    assert f(None, None, None, None, 8, 0, 128, E, 1, None) == OK


def test_noalloc_scratch_holds_every_fprop_plan(L):
    """Every FProp plan's K-split partial sums fit the allocation-free entry point's scratch:
    a split is planned only while its workgroups fit one wave over the chip (at most 256 tiles
    of 256 x 256 fp32, or of 64 rows x 64 columns on the decode kernel)."""
    cap = qr.QR_NOALLOC_SCRATCH_BYTES
    worst = 0
    for M in (1, 16, 33, 64, 65, 100, 128, 200, 256, 257, 384, 512, 1000, 2048, 8192):
        for N in (8, 200, 1024, 4096, 5120, 7168, 14336, 27648, 32512, 32768, 55296):
            for K in (128, 1024, 4096, 5120, 14336, 27648):
                nb = L.qr_gemm_workspace_bytes(0, M, N, K)
                worst = max(worst, nb)
                assert nb <= cap, (M, N, K, nb)
    assert worst > cap // 2                                           # the bound is tight


def test_rmsnorm_quant_dual_validation(L):
    f = lambda h, rows, cols, ld, g, eps, inv, y, q, s, qT, sT: L.qr_rmsnorm_quant_dual(
        h, rows, cols, ld, g, ctypes.c_float(eps), inv, y, q, s, qT, sT, None)
    assert f(A, 8, 128, 128, B, 1e-6, C, None, None, None, None, None) == NULL   # no output pair
    assert f(A, 8, 128, 128, B, 1e-6, C, None, D, None, None, None) == NULL      # half a pair
    assert f(A, 8, 128, 128, None, 1e-6, C, None, D, E, None, None) == NULL      # no gain
    assert f(A, 8, 128, 128, B, 1e-6, None, None, D, E, None, None) == NULL      # no inv_rms
    assert f(A, 12, 128, 128, B, 1e-6, C, None, None, None, D, E) == SHAPE       # colT: rows % 8
    assert f(A, 8, 100, 104, B, 1e-6, C, None, D, E, None, None) == SHAPE        # cols % 8
    assert f(A, 8, 128, 128, B, -1.0, C, None, D, E, None, None) == ARG          # eps
    assert f(A, 8, 128, 128, B + 4, 1e-6, C, None, D, E, None, None) == ALIGN    # gain 16 B
    assert f(A, 8, 128, 128, B, 1e-6, C + 2, None, D, E, None, None) == ALIGN    # inv 4 B
    assert f(A, 8, 128, 128, B, 1e-6, A + 64, None, D, E, None, None) == ALIAS   # inv inside h
    assert f(A, 8, 128, 128, B, 1e-6, C, None, D, D + 512, None, None) == ALIAS  # s inside q
    assert f(A, 0, 128, 128, B, 1e-6, C, None, D, E, None, None) == OK           # empty
