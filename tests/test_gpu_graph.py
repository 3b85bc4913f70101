"""Every entry point captured into one HIP graph (through torch.cuda.graph) and replayed: the
library allocates nothing and records no memory sets, so a captured step is a chain of kernel
nodes.  Each replay follows eager work and a garbage fill of every output, and must reproduce
the eager call's outputs bit for bit (the K-split paths included: partial sums in a caller
workspace and in the allocation-free FProp's scratch)."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_qr_amd as qr
import qr_synth
from gpu_util import dev, dev_bf16

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qr.load()


def _e(*shape, dt=torch.uint8):
    return torch.empty(shape, dtype=dt, device="cuda:0")


def _ws(kind, M, N, K):
    nb = qr.qr_gemm_workspace_bytes(kind, M, N, K)
    return (_e(nb) if nb else None), nb


def _build():
    """Inputs, outputs and the calls of one captured step (small shapes that still take every
    plan: the 256-row tiles over several row bands and in one band with early B loads and a K
    split, the decode tiles with and without a split, the batched norm paths, INT8 with a split,
    the 4-bit path)."""
    f32, bf, i8 = torch.float32, torch.bfloat16, torch.int8
    T, N, K = 640, 1024, 768                        # tokens, output features, input features
    rng = np.random.default_rng(5)
    X = dev_bf16(qr_synth.normal_bf16(41, (T, K), 1.0, 3, 7))
    dY = dev_bf16(qr_synth.normal_bf16(42, (T, N), 1e-3))
    W = dev_bf16(qr_synth.normal_bf16(43, (N, K), 0.02))
    s = dev(rng.uniform(1.5, 4.0, K).astype(np.float32))
    Wd = dev_bf16(qr_synth.normal_bf16(44, (4096, 4096), 0.02))
    Xd = dev_bf16(qr_synth.normal_bf16(45, (64, 4096), 1.0, 5, 40))
    Hs = dev_bf16(qr_synth.normal_bf16(46, (256, 1024), 1.0, 6, 10))
    gain = dev(rng.uniform(0.5, 2.0, 1024).astype(np.float32))
    Xb = dev_bf16(qr_synth.normal_bf16(47, (200, 512), 1.0))
    Wb = dev_bf16(qr_synth.normal_bf16(48, (9000, 512), 0.02))
    X8 = dev_bf16(qr_synth.normal_bf16(49, (200, 2048), 1.0))
    W8 = dev_bf16(qr_synth.normal_bf16(50, (1000, 2048), 0.02))
    Xn = dev_bf16(qr_synth.normal_bf16(51, (200, 1024), 1.0))
    Wn = dev_bf16(qr_synth.normal_bf16(52, (4096, 1024), 0.02))
    X4 = dev_bf16(qr_synth.normal_bf16(53, (64, 1024), 1.0))
    W4 = dev_bf16(qr_synth.normal_bf16(54, (1000, 1024), 0.02))
    Xs = dev_bf16(qr_synth.normal_bf16(55, (200, 8192), 1.0))
    Ws = dev_bf16(qr_synth.normal_bf16(56, (4096, 8192), 0.02))

    o = {}
    o["Wf"], o["qW"], o["sW"] = _e(N, K, dt=bf), _e(N, K), _e(N // 128, K // 128, dt=f32)
    o["qWT"], o["sWT"] = _e(K, N), _e(K // 128, N // 128, dt=f32)
    o["qX"], o["sX"], o["qXT"], o["sXT"] = _e(T, K), _e(T, K // 128, dt=f32), _e(K, T), _e(K, T // 128, dt=f32)
    o["qdY"], o["sdY"], o["qdYT"], o["sdYT"] = _e(T, N), _e(T, N // 128, dt=f32), _e(N, T), _e(N, T // 128, dt=f32)
    o["Y"], o["dX"], o["dW"] = _e(T, N, dt=bf), _e(T, K, dt=bf), _e(N, K, dt=f32)
    o["qWd"], o["sWd"] = _e(4096, 4096), _e(32, 32, dt=f32)
    o["qXd"], o["sXd"], o["Yd"] = _e(64, 4096), _e(64, 32, dt=f32), _e(64, 4096, dt=bf)
    o["yH"], o["qH"], o["sH"] = _e(256, 1024, dt=bf), _e(256, 1024), _e(256, 8, dt=f32)
    o["inv"], o["qH2"], o["sH2"], o["qH2T"], o["sH2T"] = (_e(256, dt=f32), _e(256, 1024), _e(256, 8, dt=f32),
                                                          _e(1024, 256), _e(1024, 2, dt=f32))
    o["qXb"], o["sXb"], o["qWb"], o["sWb"], o["Yb"] = (_e(200, 512), _e(200, 4, dt=f32), _e(9000, 512),
                                                       _e(71, 4, dt=f32), _e(200, 9000, dt=bf))
    o["qX8"], o["sX8"], o["qW8"], o["sW8"], o["Y8"] = (_e(200, 2048, dt=i8), _e(200, dt=f32),
                                                       _e(1000, 2048, dt=i8), _e(1000, dt=f32),
                                                       _e(200, 1000, dt=f32))
    o["qXn"], o["sXn"], o["qWn"], o["sWn"], o["Yn"] = (_e(200, 1024), _e(200, 8, dt=f32), _e(4096, 1024),
                                                       _e(32, 8, dt=f32), _e(200, 4096, dt=bf))
    o["c4"], o["b4"], o["t4"], o["Y4"] = (_e(1000, 512), _e(1000, 64), _e(1, dt=f32),
                                          _e(64, 1000, dt=bf))
    o["qXs"], o["sXs"], o["qWs"], o["sWs"], o["Ys"] = (_e(200, 8192), _e(200, 64, dt=f32), _e(4096, 8192),
                                                       _e(32, 64, dt=f32), _e(200, 4096, dt=bf))
    ws = {"fprop": _ws(qr.QR_GEMM_FPROP, T, N, K), "dgrad": _ws(qr.QR_GEMM_DGRAD, T, N, K),
          "wgrad": _ws(qr.QR_GEMM_WGRAD, T, N, K), "dec": _ws(qr.QR_GEMM_FPROP, 64, 4096, 4096),
          "band": _ws(qr.QR_GEMM_FPROP, 200, 9000, 512), "i8": _ws(qr.QR_GEMM_INT8, 200, 1000, 2048),
          "split": _ws(qr.QR_GEMM_FPROP, 200, 4096, 8192)}
    ws4 = _e(qr.QR_NVFP4_WORKSPACE_BYTES)
    # split paths: the decode tiles (64 rows), 256x128 tiles (one row band, 8 splits), INT8
    assert ws["dec"][1] > 0 and ws["split"][1] > 0 and ws["i8"][1] > 0, "split paths expected"
    assert ws["band"][1] == 0, "one row band, unsplit, expected"
    BF, F32 = qr.QR_OUT_BF16, qr.QR_OUT_F32

    def step():
        qr.qr_uaq_fold_quant_w_128x128(W, N, K, K, s, o["Wf"], None, o["qW"], o["sW"], o["qWT"], o["sWT"])
        qr.qr_quant_act_1x128(X, T, K, K, o["qX"], o["sX"], o["qXT"], o["sXT"])
        qr.qr_gemm_fp8_bsfprop(o["qX"], o["sX"], o["qW"], o["sW"], T, N, K, o["Y"], BF, *ws["fprop"])
        qr.qr_quant_act_1x128(dY, T, N, N, o["qdY"], o["sdY"], o["qdYT"], o["sdYT"])
        qr.qr_gemm_fp8_bsdgrad(o["qdY"], o["sdY"], o["qWT"], o["sWT"], T, N, K, o["dX"], BF, *ws["dgrad"])
        qr.qr_gemm_fp8_bswgrad(o["qdYT"], o["sdYT"], o["qXT"], o["sXT"], T, N, K, o["dW"], F32, *ws["wgrad"])
        qr.qr_quant_w_128x128(Wd, 4096, 4096, 4096, o["qWd"], o["sWd"], None, None)
        qr.qr_rmsnorm_quant_1x128(Xd, 64, 4096, 4096, o["gain_d"], 1e-6, None, o["qXd"], o["sXd"])
        qr.qr_gemm_fp8_bsfprop(o["qXd"], o["sXd"], o["qWd"], o["sWd"], 64, 4096, 4096, o["Yd"], BF, *ws["dec"])
        qr.qr_rmsnorm_quant_1x128(Hs, 256, 1024, 1024, gain, 1e-6, o["yH"], o["qH"], o["sH"])
        qr.qr_rmsnorm_quant_dual(Hs, 256, 1024, 1024, gain, 1e-6, o["inv"], None, o["qH2"], o["sH2"],
                                 o["qH2T"], o["sH2T"])
        qr.qr_quant_act_1x128(Xb, 200, 512, 512, o["qXb"], o["sXb"], None, None)
        qr.qr_quant_w_128x128(Wb, 9000, 512, 512, o["qWb"], o["sWb"], None, None)
        qr.qr_gemm_fp8_bsfprop(o["qXb"], o["sXb"], o["qWb"], o["sWb"], 200, 9000, 512, o["Yb"], BF, *ws["band"])
        qr.qr_quant_int8_rowwise(X8, 200, 2048, 2048, o["qX8"], o["sX8"])
        qr.qr_quant_int8_rowwise(W8, 1000, 2048, 2048, o["qW8"], o["sW8"])
        qr.qr_gemm_int8_w8a8(o["qX8"], o["sX8"], o["qW8"], o["sW8"], 200, 1000, 2048, o["Y8"], F32, *ws["i8"])
        qr.qr_quant_act_1x128(Xn, 200, 1024, 1024, o["qXn"], o["sXn"], None, None)
        qr.qr_quant_w_128x128(Wn, 4096, 1024, 1024, o["qWn"], o["sWn"], None, None)
        qr.qr_gemm_fp8_bsfprop_noalloc(o["qXn"], o["sXn"], o["qWn"], o["sWn"], 200, 4096, 1024, o["Yn"], BF)
        qr.qr_quant_w_nvfp4(W4, 1000, 1024, 1024, o["c4"], o["b4"], o["t4"], ws4,
                            qr.QR_NVFP4_WORKSPACE_BYTES)
        qr.qr_gemm_w4a16(X4, o["c4"], o["b4"], o["t4"], 64, 1000, 1024, o["Y4"], BF)
        qr.qr_quant_act_1x128(Xs, 200, 8192, 8192, o["qXs"], o["sXs"], None, None)
        qr.qr_quant_w_128x128(Ws, 4096, 8192, 8192, o["qWs"], o["sWs"], None, None)
        qr.qr_gemm_fp8_bsfprop(o["qXs"], o["sXs"], o["qWs"], o["sWs"], 200, 4096, 8192, o["Ys"], BF, *ws["split"])

    o["gain_d"] = dev(np.full(4096, 1.25, np.float32))
    outputs = [k for k in o if k != "gain_d"]
    return step, o, outputs


def _snapshot(o, names):
    torch.cuda.synchronize()
    return {k: o[k].detach().clone() for k in names}


def _garble(o, names, seed):
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    for k in names:
        bits = o[k].view(torch.uint8)
        bits.copy_(torch.randint(0, 256, bits.shape, dtype=torch.uint8, device="cuda:0", generator=g))


def _same(a, b):
    return np.array_equal(a.view(torch.uint8).cpu().numpy(), b.view(torch.uint8).cpu().numpy())


def test_graph_replays_match_eager():
    step, o, outputs = _build()
    step()                                   # eager reference
    ref = _snapshot(o, outputs)
    step()                                   # eager again: the calls are deterministic
    again = _snapshot(o, outputs)
    for k in outputs:
        assert _same(ref[k], again[k]), f"{k}: two eager calls differ"

    side = torch.cuda.Stream()               # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                               # warm-up on the capture's side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 22, device="cuda:0")
    for rep in range(3):
        _garble(o, outputs, 100 + rep)       # every output overwritten before the replay
        scratch.mul_(1.0001).sum()           # the program's own eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in outputs:
            assert _same(o[k], ref[k]), f"replay {rep}: {k} differs from the eager call"
        print(f"[graph] replay {rep}: {len(outputs)} outputs equal to the eager call", flush=True)
    del graph
