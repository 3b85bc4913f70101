"""The allocation-free FProp (qr_gemm_fp8_bsfprop_noalloc) through the C ABI against the
workspace entry point (qr_gemm_fp8_bsfprop): bit-identical outputs, on two calls in a row
with the second smaller, for plans with and without a K split and both output types."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_qr_amd as qr
import oracle
import qr_synth
from gpu_util import dev, dev_bf16, g_quant_act, g_quant_w, guarded_empty

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qr.load()


def _operands(M, N, K, seed):
    x = qr_synth.normal_bf16(seed, (M, K), 1.0, seed + 1, max(1, K // 100))
    w = qr_synth.normal_bf16(seed + 2, (N, K), 0.02)
    qa, sa, _, _ = g_quant_act(qr, dev_bf16(x), row=True)
    if N % 8 == 0:
        qw, sw, _, _ = g_quant_w(qr, dev_bf16(w))
    else:
        # the weight quantizer takes n % 8 == 0; such a weight's codes come from the oracle
        rw, rsw = oracle.quant_blocks(w)
        qw, sw = dev(rw), dev(rsw)
    return qa, sa, qw, sw


def _both(M, N, K, seed, out):
    qa, sa, qw, sw = _operands(M, N, K, seed)
    dt = torch.bfloat16 if out == qr.QR_OUT_BF16 else torch.float32
    nb = qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, M, N, K)
    checks = []
    y_ref = guarded_empty((M, N), dt, checks)
    ws = guarded_empty((nb,), torch.uint8, checks) if nb else None
    qr.qr_gemm_fp8_bsfprop(qa, sa, qw, sw, M, N, K, y_ref, out, ws, nb)
    y = guarded_empty((M, N), dt, checks)
    qr.qr_gemm_fp8_bsfprop_noalloc(qa, sa, qw, sw, M, N, K, y, out)
    for c in checks:
        c()
    return nb, y, y_ref


# (large, then smaller): 32B QKV at batch 256 (4 K splits on 256x128 tiles, 29 MB of partials)
# then the 8B O projection at batch 64 (4 splits, 4 MB); a 2-split decode then an unsplit one;
# a ragged split of 201 rows on the 64-row tiles (odd M * N, 2 splits) then a smaller unsplit
# ragged one
PAIRS = [((256, 7168, 5120), (64, 4096, 4096)),
         ((64, 1000, 2304), (16, 200, 384)),
         ((201, 77, 2048), (77, 77, 384))]


@pytest.mark.parametrize("first,second", PAIRS)
@pytest.mark.parametrize("out", [qr.QR_OUT_F32, qr.QR_OUT_BF16])
def test_noalloc_matches_workspace_entry(first, second, out):
    for i, (M, N, K) in enumerate((first, second)):
        print("[case] noalloc", M, N, K, "out", out, flush=True)
        nb, y, y_ref = _both(M, N, K, 7 * M + N + i, out)
        if i == 0:
            assert nb > 0, "the first call of each pair takes a K split"
        assert torch.equal(y.view(torch.uint8), y_ref.view(torch.uint8)), (M, N, K, out)
