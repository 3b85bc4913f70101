#!/usr/bin/env python3
"""Benchmark of the MI355X FP8 quantize-and-multiply path (one GPU).

One step is one pass of the whole linear-layer path over one batch of seeded synthetic
input, at the 8B-layer shapes (hidden 4096, 8192 tokens; decode FFN 14336 at batch 64):

  fold_quant_w    W' = W [4096, 4096] / s (per input column), gain * s, and the 128x128
                  blocks of W' plus the transposed copy for DGrad, in one pass over W
                  (the fold is a one-time op; timed)
  quant_x_dual    1x128 rows of X [8192, 4096] for FProp and its 128x1 columns (transposed)
                  for WGrad, one read (X is the norm output carrying s); the column codes are
                  the FP8 activations kept for the backward
  fprop           Y = X W^T            8192 x 4096 x 4096, bf16 out
  quant_dy_dual   1x128 rows and 128x1 columns (transposed) of dY [8192, 4096], one read
  dgrad           dX = dY W            8192 x 4096 x 4096, bf16 out
  wgrad           dW = dY^T X          4096 x 4096 x 8192, bf16 out
  quant_x_dec     1x128 groups of the decode activation X [64, 4096]
  fprop_decode    Y = X W^T            64 x 14336 x 4096 on the pre-quantized weight, bf16 out

After the warm-up, a breakdown pass of K steps brackets every launch with HIP events on the
stream it runs on (each op's time and roofline fraction).  The timed pass of K steps then
records events only around the dominant kernel's launch, so the step time carries no per-op
event overhead.  The JSON line reports the step's GEMM throughput (all GEMM flops / step
time) as `value`, each op's time with its roofline fraction, the roofline of the dominant
kernel from its launches in the timed pass, and the CPU oracle timed on a bounded token slice
of the same step.  Outside the step it also times the batched re-quantization of a 32B
decoder layer's four weights (`weight_update`, once per optimizer step), the norm with the
activation quantize fused in (`norm_quant`, the producer of FProp's operand), the INT8
W8A8 variant at the same shapes (`int8_w8a8`), the 4-bit weight path at the decode shape
(`w4a16`: quantizing the 14336x4096 weight, then the 64x14336x4096 GEMM with bf16 X) and the
8B decoder layer's four FP8 linears at decode batch 64 (`decode_8b`) and the 32B decoder
layer's four at decode batch 256 on the weight update's codes (`decode_32b`).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_INT8_TOPS = 5000.0     # MI355X dense INT8 MFMA
METRIC = "FP8 block-scaled GEMM TFLOP/s (% FP8 MFMA peak) + quantize GB/s (% HBM)"

T, H, F, MD = 8192, 4096, 14336, 64     # tokens, hidden, decode FFN width, decode batch


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gemm_flops(m, n, k):
    return 2.0 * m * n * k


def op_table():
    """Algorithmic work of each op: ('mfma', flops) or ('hbm', bytes), minimum traffic."""
    g = 128
    return {
        # read W bf16 + s + gain; write W' bf16 + gain, codes twice + block scales twice
        "fold_quant_w": ("hbm", H * H * 2 * 2 + H * 4 * 3 + 2 * H * H + 2 * (H // g) ** 2 * 4),
        # read X once, write row codes + scales and transposed column codes + scales
        "quant_x_dual": ("hbm", T * H * 2 + 2 * T * H + T * (H // g) * 4 + H * (T // g) * 4),
        "fprop": ("mfma", gemm_flops(T, H, H)),
        "quant_dy_dual": ("hbm", T * H * 2 + 2 * T * H + 2 * T * (H // g) * 4),
        "dgrad": ("mfma", gemm_flops(T, H, H)),
        "wgrad": ("mfma", gemm_flops(H, H, T)),
        "quant_x_dec": ("hbm", MD * H * 2 + MD * H + MD * (H // g) * 4),
        # decode is bound by streaming the weight: codes + block scales + A + Y
        "fprop_decode": ("hbm", F * H + (F // g) * (H // g) * 4 + MD * H + MD * (H // g) * 4
                         + MD * F * 2),
    }


def decode_flops():
    return gemm_flops(MD, F, H)


# Sources each op's kernels are built from (a traffic figure is valid only for these).
GEMM_SOURCES = ("gemm.hip", "qr_device.h", "qr_internal.h")
QUANT_SOURCES = ("quant.hip", "qr_device.h", "qr_internal.h")


def kernel_source_sha(kernel="wgrad"):
    files = GEMM_SOURCES if op_table()[kernel][0] == "mfma" or "decode" in kernel else QUANT_SOURCES
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "fp8_block_scaled_qr_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(kernel)
    if not e or e.get("source_sha") != kernel_source_sha(kernel):
        return None
    return e.get("bytes_per_launch")


# ------------------------------------------------------------------ GPU part

class Step:
    def __init__(self, torch, qr):
        import qr_synth
        self.torch, self.qr = torch, qr
        dev = "cuda:0"
        t0 = time.time()
        s = qr_synth.uniform_f32(3011, H, 1.5, 4.0)
        x = qr_synth.normal_bf16(3001, (T, H), 1.0, 3003, qr_synth.n_outliers(H), col_scale=s)
        w = qr_synth.normal_bf16(3002, (H, H), 0.02)
        dy = qr_synth.backward_8b_dy()
        dec = qr_synth.decode_8b()
        xd, wd = dec.x(), dec.w()
        log(f"inputs generated in {time.time() - t0:.1f}s")

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        u8, f32 = torch.uint8, torch.float32
        self.X, self.W, self.dY, self.Xd = bf(x), bf(w), bf(dy), bf(xd)
        self.s = torch.from_numpy(s).to(dev)
        self.gain = torch.ones(H, dtype=f32, device=dev)
        e = lambda *sh, dt=u8: torch.empty(sh, dtype=dt, device=dev)
        g = 128
        self.Wf = torch.empty_like(self.W)
        self.qW, self.sW, self.qWT, self.sWT = e(H, H), e(H // g, H // g, dt=f32), e(H, H), e(H // g, H // g, dt=f32)
        self.qX, self.sX = e(T, H), e(T, H // g, dt=f32)
        self.Y = e(T, H, dt=torch.bfloat16)
        self.qdY, self.sdY, self.qdYT, self.sdYT = e(T, H), e(T, H // g, dt=f32), e(H, T), e(H, T // g, dt=f32)
        self.qXT, self.sXT = e(H, T), e(H, T // g, dt=f32)
        self.dX, self.dW = e(T, H, dt=torch.bfloat16), e(H, H, dt=torch.bfloat16)
        self.qXd, self.sXd = e(MD, H), e(MD, H // g, dt=f32)
        self.Yd = e(MD, F, dt=torch.bfloat16)
        # the decode weight is quantized once, outside the step (weights change per update)
        Wd = bf(wd)
        self.qWd, self.sWd = e(F, H), e(F // g, H // g, dt=f32)
        qr.qr_quant_w_128x128(Wd, F, H, H, self.qWd, self.sWd, None, None)
        del Wd
        self.ws = {}
        for kind, (M, N, K) in (("fprop", (T, H, H)), ("dgrad", (T, H, H)), ("wgrad", (T, H, H)),
                                ("decode", (MD, F, H))):
            code = {"fprop": 0, "dgrad": 1, "wgrad": 2, "decode": 0}[kind]
            nb = qr.qr_gemm_workspace_bytes(code, M, N, K)
            self.ws[kind] = (e(nb) if nb else None, nb)
        torch.cuda.synchronize()

    def ops(self):
        qr, BF = self.qr, self.qr.QR_OUT_BF16
        return [
            ("fold_quant_w", lambda: qr.qr_uaq_fold_quant_w_128x128(
                self.W, H, H, H, self.s, self.Wf, self.gain, self.qW, self.sW, self.qWT, self.sWT)),
            ("quant_x_dual", lambda: qr.qr_quant_act_1x128(self.X, T, H, H, self.qX, self.sX, self.qXT,
                                                           self.sXT)),
            ("fprop", lambda: qr.qr_gemm_fp8_bsfprop(self.qX, self.sX, self.qW, self.sW, T, H, H, self.Y, BF,
                                                     *self.ws["fprop"])),
            ("quant_dy_dual", lambda: qr.qr_quant_act_1x128(self.dY, T, H, H, self.qdY, self.sdY, self.qdYT,
                                                            self.sdYT)),
            ("dgrad", lambda: qr.qr_gemm_fp8_bsdgrad(self.qdY, self.sdY, self.qWT, self.sWT, T, H, H, self.dX, BF,
                                                     *self.ws["dgrad"])),
            ("wgrad", lambda: qr.qr_gemm_fp8_bswgrad(self.qdYT, self.sdYT, self.qXT, self.sXT, T, H, H, self.dW, BF,
                                                     *self.ws["wgrad"])),
            ("quant_x_dec", lambda: qr.qr_quant_act_1x128(self.Xd, MD, H, H, self.qXd, self.sXd, None, None)),
            ("fprop_decode", lambda: qr.qr_gemm_fp8_bsfprop(self.qXd, self.sXd, self.qWd, self.sWd, MD, F, H,
                                                            self.Yd, BF, *self.ws["decode"])),
        ]


def run_gpu(args):
    import torch
    import fp8_block_scaled_qr_amd as qr
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (MI355X)")
    qr.load()
    torch.cuda.set_device(0)
    st = Step(torch, qr)
    ops = st.ops()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for _, f in ops:
            f()
    torch.cuda.synchronize()

    def events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(n)]

    # Per-op breakdown: its own pass of K steps with an event pair around every launch (the
    # event records add a few microseconds per launch, so this pass is not the timed one).
    ev = [events(len(ops)) for _ in range(args.steps)]
    for k in range(args.steps):
        for (name, f), (a, b) in zip(ops, ev[k]):
            a.record(stream)
            f()
            b.record(stream)
    torch.cuda.synchronize()
    per_op = {name: float(np.mean([ev[k][i][0].elapsed_time(ev[k][i][1])
                                   for k in range(args.steps)]))
              for i, (name, _) in enumerate(ops)}
    dom = max(per_op, key=lambda n: per_op[n])

    # Timed region: K steps; events only around the dominant kernel's launch in each step.
    dev_ev = events(args.steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        for name, f in ops:
            if name == dom:
                dev_ev[k][0].record(stream)
                f()
                dev_ev[k][1].record(stream)
            else:
                f()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(end) / args.steps
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in dev_ev]))
    normq = run_norm_quant(torch, qr, st)
    int8 = run_int8(torch, qr, st)
    w4 = run_w4a16(torch, qr, st)
    del st, ops
    torch.cuda.empty_cache()
    dec8 = run_decode_8b(torch, qr)
    torch.cuda.empty_cache()
    upd, codes = run_weight_update(torch, qr)
    dec32 = run_decode_32b(torch, qr, codes)
    del codes
    torch.cuda.empty_cache()
    return step_ms, wall, per_op, dom, dom_ms, upd, normq, int8, w4, dec8, dec32


def run_norm_quant(torch, qr, st, iters=20):
    """The norm in front of FProp with its 1x128 quantization fused in, on the prefill hidden
    state [8192, 4096] (the step's X stands in for h; the gain carries the UAQ s), writing the
    FProp operand only (codes and scales): 2 + 1 + 4/128 bytes per element."""
    dev = "cuda:0"
    g = st.s.clone()
    q = torch.empty((T, H), dtype=torch.uint8, device=dev)
    s = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    f = lambda: qr.qr_rmsnorm_quant_1x128(st.X, T, H, H, g, 1e-6, None, q, s)
    us = _median_us(torch, f, iters)
    nbytes = T * H * 2 + T * H + T * (H // 128) * 4 + H * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "RMSNorm (gain carrying the UAQ s) + 1x128 quantize of h [8192, 4096], "
                        "codes and scales out (the FProp operand)",
            "us": round(us, 2), "bound": "hbm", "bytes": nbytes, "achieved": round(gbs, 1),
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}


_FLUSH = None


def _median_us(torch, f, iters, flush=True):
    """Median event time of f() on the current stream.  With flush, a 512 MiB buffer is read
    before each call (outside the events; reading leaves no dirty lines to write back during
    the timed call), so inputs that would fit the 256 MB MALL come from HBM."""
    global _FLUSH
    if flush and _FLUSH is None:
        _FLUSH = torch.ones(128 << 20, dtype=torch.float32, device="cuda:0")
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        if flush:
            _FLUSH.sum()
        a.record(stream)
        f()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3


def run_int8(torch, qr, st, iters=20):
    """The INT8 W8A8 variant at the same shapes: the per-token quantize of X [8192, 4096], the
    prefill GEMM 8192x4096x4096 and the decode GEMM 64x14336x4096 (bf16 out), then the 32B
    layer's four linears at decode batch 256."""
    dev = "cuda:0"
    e = lambda *sh, dt: torch.empty(sh, dtype=dt, device=dev)
    i8, f32, bf = torch.int8, torch.float32, torch.bfloat16
    qx, sx = e(T, H, dt=i8), e(T, dt=f32)
    qw, sw = e(H, H, dt=i8), e(H, dt=f32)
    qr.qr_quant_int8_rowwise(st.W, H, H, H, qw, sw)
    g = torch.Generator(device=dev).manual_seed(7001)
    wd = (torch.randn((F, H), device=dev, generator=g) * 0.02).to(bf)
    qwd, swd = e(F, H, dt=i8), e(F, dt=f32)
    qr.qr_quant_int8_rowwise(wd, F, H, H, qwd, swd)
    del wd
    qxd, sxd = e(MD, H, dt=i8), e(MD, dt=f32)
    qr.qr_quant_int8_rowwise(st.Xd, MD, H, H, qxd, sxd)
    y, yd = e(T, H, dt=bf), e(MD, F, dt=bf)
    out = {}
    us = _median_us(torch, lambda: qr.qr_quant_int8_rowwise(st.X, T, H, H, qx, sx), iters)
    nb = T * H * 3 + T * 4
    out["quant_x"] = {"us": round(us, 2), "bound": "hbm", "bytes": nb,
                      "achieved": round(nb / us / 1e3, 1), "unit": "GB/s",
                      "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    us = _median_us(torch, lambda: qr.qr_gemm_int8_w8a8(qx, sx, qw, sw, T, H, H, y, 1), iters)
    tops = 2.0 * T * H * H / (us * 1e-6) / 1e12
    out["gemm_prefill"] = {"shape": [T, H, H], "us": round(us, 2), "bound": "mfma",
                           "achieved": round(tops, 1), "unit": "TOP/s",
                           "frac": round(tops / PEAK_INT8_TOPS, 4)}
    us = _median_us(torch, lambda: qr.qr_gemm_int8_w8a8(qxd, sxd, qwd, swd, MD, F, H, yd, 1), iters)
    nb = F * H + F * 4 + MD * H + MD * 4 + MD * F * 2
    out["gemm_decode"] = {"shape": [MD, F, H], "us": round(us, 2), "bound": "hbm", "bytes": nb,
                          "achieved": round(nb / us / 1e3, 1), "unit": "GB/s",
                          "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    del qwd, swd, qxd, sxd, yd
    out["layer_32b_batch256"] = run_int8_32b(torch, qr, iters)
    return out


def run_int8_32b(torch, qr, iters):
    """The 32B decoder layer's four linears at decode batch 256 in INT8 W8A8 (random codes
    and positive scales; the GEMM's time does not depend on the values), bf16 out, each after
    a cache-evicting read.  Algorithmic bytes = weight codes and scales + activation codes and
    scales + bf16 Y."""
    dev = "cuda:0"
    M = 256
    shapes = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 55296, 5120),
              ("down", 5120, 27648)]
    gen = torch.Generator(device=dev).manual_seed(6301)
    out, tot_us, tot_b = {}, 0.0, 0
    for name, n, k in shapes:
        qw = torch.randint(-127, 127, (n, k), dtype=torch.int8, device=dev, generator=gen)
        sw = torch.rand((n,), device=dev, generator=gen) * 1e-3 + 1e-4
        qx = torch.randint(-127, 127, (M, k), dtype=torch.int8, device=dev, generator=gen)
        sx = torch.rand((M,), device=dev, generator=gen) * 1e-2 + 1e-3
        y = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        nb = qr.qr_gemm_workspace_bytes(qr.QR_GEMM_INT8, M, n, k)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        us = _median_us(torch, lambda: qr.qr_gemm_int8_w8a8(qx, sx, qw, sw, M, n, k, y,
                                                           qr.QR_OUT_BF16, ws, nb), iters)
        by = n * k + n * 4 + M * k + M * 4 + M * n * 2
        gbs = by / (us * 1e-6) / 1e9
        out[name] = {"shape": [M, n, k], "us": round(us, 2), "gbs": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                     "k_splits": nb // (M * n * 4) if nb else 1}
        tot_us, tot_b = tot_us + us, tot_b + by
        del qw, sw, qx, sx, y, ws
    out["layer"] = {"us": round(tot_us, 1), "gbs": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
                    "frac_hbm": round(tot_b / (tot_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    out["workload"] = ("32B decoder layer at decode batch 256, INT8 W8A8: QKV 5120->7168, "
                       "O 5120->5120, gate+up 5120->55296, down 27648->5120")
    return out


def run_w4a16(torch, qr, st, iters=20):
    """The 4-bit weight path at the decode shape: NVFP4-style quantization of the 14336x4096
    weight (E2M1 codes, an E4M3 scale per 16, an fp32 tensor scale; two passes, the first for
    the tensor's amax) and the decode GEMM 64x14336x4096 with bf16 X (bf16 out)."""
    dev = "cuda:0"
    u8 = torch.uint8
    g = torch.Generator(device=dev).manual_seed(7002)
    wd = (torch.randn((F, H), device=dev, generator=g) * 0.02).to(torch.bfloat16)
    codes = torch.empty((F, H // 2), dtype=u8, device=dev)
    bs = torch.empty((F, H // 16), dtype=u8, device=dev)
    t = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(qr.QR_NVFP4_WORKSPACE_BYTES, dtype=u8, device=dev)
    yd = torch.empty((MD, F), dtype=torch.bfloat16, device=dev)
    out = {}
    us = _median_us(torch, lambda: qr.qr_quant_w_nvfp4(wd, F, H, H, codes, bs, t, ws,
                                                       qr.QR_NVFP4_WORKSPACE_BYTES), iters)
    nb = F * H * 2 + F * H // 2 + F * H // 16 + 4
    out["quant_w"] = {"shape": [F, H], "us": round(us, 2), "bound": "hbm", "bytes": nb,
                      "achieved": round(nb / us / 1e3, 1), "unit": "GB/s",
                      "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    del wd
    us = _median_us(torch, lambda: qr.qr_gemm_w4a16(st.Xd, codes, bs, t, MD, F, H, yd, 1), iters)
    nb = F * H // 2 + F * H // 16 + 4 + MD * H * 2 + MD * F * 2
    out["gemm_decode"] = {"shape": [MD, F, H], "us": round(us, 2), "bound": "hbm", "bytes": nb,
                          "achieved": round(nb / us / 1e3, 1), "unit": "GB/s",
                          "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    return out


def run_weight_update(torch, qr, iters=10):
    """Quantize-on-update of the 32B decoder layer's four weights (QKV, O, gate+up, down),
    each with its transposed copy, as one batched call; timed outside the step (it runs once
    per optimizer step, not per token).  Inputs: seeded N(0, 0.02) on the device."""
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(6001)
    shapes = [(7168, 5120), (5120, 5120), (55296, 5120), (5120, 27648)]
    ws = [(torch.randn(sh, device=dev, generator=g) * 0.02).to(torch.bfloat16) for sh in shapes]
    items = []
    nbytes = 0
    for w in ws:
        n, k = w.shape
        nb = ((n + 127) // 128) * ((k + 127) // 128)
        q = torch.empty((n, k), dtype=torch.uint8, device=dev)
        qT = torch.empty((k, n), dtype=torch.uint8, device=dev)
        s = torch.empty(nb, dtype=torch.float32, device=dev)
        sT = torch.empty(nb, dtype=torch.float32, device=dev)
        items.append((w, n, k, k, q, s, qT, sT))
        nbytes += n * k * (2 + 1 + 1) + 2 * nb * 4
    us = _median_us(torch, lambda: qr.qr_quant_w_128x128_batched(items), iters, flush=False)
    gbs = nbytes / (us * 1e-6) / 1e9
    codes = [(q, s, n, k) for (_, n, k, _, q, s, _, _) in items]
    del ws, items
    torch.cuda.empty_cache()
    upd = {"workload": "32B decoder layer weights (QKV 7168x5120, O 5120x5120, gate+up "
                       "55296x5120, down 5120x27648) re-quantized 128x128 with transposed "
                       "copies, one batched call",
           "us": round(us, 1), "bound": "hbm", "bytes": nbytes, "achieved": round(gbs, 1),
           "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "launches": 1}
    return upd, codes


def run_decode_8b(torch, qr, iters=20):
    """The 8B decoder layer's four linears at decode batch 64 (QKV 4096->6144, O 4096->4096,
    gate+up 4096->28672, down 14336->4096): seeded N(0, 0.02) weights quantized 128x128, then
    FProp on 1x128 activation codes, bf16 out, each after a cache-evicting read."""
    dev = "cuda:0"
    M, g = MD, 128
    shapes = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096),
              ("down", 4096, 14336)]
    gen = torch.Generator(device=dev).manual_seed(6201)
    out, tot_us, tot_b = {}, 0.0, 0
    for name, n, k in shapes:
        w = (torch.randn((n, k), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        q, s = qr.quant_w(w)[:2]
        del w
        x = torch.randn((M, k), device=dev, generator=gen).to(torch.bfloat16)
        qx, sx = qr.quant_act(x)[:2]
        y = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        nb = qr.qr_gemm_workspace_bytes(0, M, n, k)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        us = _median_us(torch, lambda: qr.qr_gemm_fp8_bsfprop(qx, sx, q, s, M, n, k, y,
                                                             qr.QR_OUT_BF16, ws, nb), iters)
        by = n * k + (n // g) * (k // g) * 4 + M * k + M * (k // g) * 4 + M * n * 2
        gbs = by / (us * 1e-6) / 1e9
        out[name] = {"shape": [M, n, k], "us": round(us, 2), "gbs": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "k_splits": nb // (M * n * 4) if nb else 1}
        tot_us, tot_b = tot_us + us, tot_b + by
        del q, s, x, qx, sx, y, ws
    out["layer"] = {"us": round(tot_us, 1), "gbs": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
                    "frac_hbm": round(tot_b / (tot_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    out["workload"] = ("8B decoder layer at decode batch 64: QKV 4096->6144, O 4096->4096, "
                       "gate+up 4096->28672, down 14336->4096; FP8 FProp, bf16 out, each after "
                       "a cache-evicting read")
    return out


def run_decode_32b(torch, qr, codes, iters=20):
    """The 32B decoder layer's four linears at decode batch 256 on their 128x128 FP8 codes
    (the weight update's output): 1x128 activation codes of X [256, K], then FProp with bf16
    out.  Each GEMM is timed after a cache-evicting read, so its weight streams from HBM.
    Algorithmic bytes = weight codes + block scales + activation codes and scales + bf16 Y."""
    dev = "cuda:0"
    M, g = 256, 128
    names = ["qkv", "o", "gate_up", "down"]
    gen = torch.Generator(device=dev).manual_seed(6101)
    out, tot_us, tot_fl, tot_b = {}, 0.0, 0.0, 0
    for name, (q, s, n, k) in zip(names, codes):
        x = torch.randn((M, k), device=dev, generator=gen).to(torch.bfloat16)
        qx, sx = qr.quant_act(x)[:2]
        y = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        nb = qr.qr_gemm_workspace_bytes(0, M, n, k)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        us = _median_us(torch, lambda: qr.qr_gemm_fp8_bsfprop(qx, sx, q, s, M, n, k, y,
                                                             qr.QR_OUT_BF16, ws, nb), iters)
        fl = gemm_flops(M, n, k)
        by = n * k + (n // g) * (k // g) * 4 + M * k + M * (k // g) * 4 + M * n * 2
        tf, gbs = fl / (us * 1e-6) / 1e12, by / (us * 1e-6) / 1e9
        out[name] = {"shape": [M, n, k], "us": round(us, 2), "tflops": round(tf, 1),
                     "gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                     "frac_mfma": round(tf / PEAK_FP8_TFLOPS, 4)}
        tot_us, tot_fl, tot_b = tot_us + us, tot_fl + fl, tot_b + by
        del x, qx, sx, y, ws
    out["layer"] = {"us": round(tot_us, 1), "tflops": round(tot_fl / (tot_us * 1e-6) / 1e12, 1),
                    "gbs": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
                    "frac_hbm": round(tot_b / (tot_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    out["workload"] = ("32B decoder layer at decode batch 256: QKV 5120->7168, O 5120->5120, "
                       "gate+up 5120->55296, down 27648->5120; FP8 FProp, bf16 out, each "
                       "after a cache-evicting read")
    return out


# ------------------------------------------------------------------ CPU oracle baseline

def run_cpu_baseline(tokens):
    """The oracle (plain C, fp64 products) on a token slice of the same step: the fold and
    quantization of the full weight, the activation/gradient quantizers and all four GEMMs
    restricted to `tokens` tokens (WGrad contracts over them; the decode GEMM keeps 64 rows
    x 1/8 of the FFN outputs)."""
    import oracle
    import qr_synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    s = qr_synth.uniform_f32(3011, H, 1.5, 4.0)
    x = qr_synth.normal_bf16(3001, (T, H), 1.0, 3003, qr_synth.n_outliers(H), col_scale=s)[:tokens]
    w = qr_synth.normal_bf16(3002, (H, H), 0.02)
    dy = qr_synth.backward_8b_dy()[:tokens]
    dec = qr_synth.decode_8b()
    xd, wd = dec.x(), dec.w()[: F // 8]
    oracle.lib()
    t0 = time.perf_counter()
    wf, _ = oracle.uaq_fold(w, s, np.ones(H, np.float32))
    qw, sw = oracle.quant_blocks(wf)
    qx, sx = oracle.quant_rows(x)
    oracle.fprop(qx, sx, qw, sw)
    qd, sd = oracle.quant_rows(dy)
    qdT, sdT = oracle.quant_cols_T(dy)
    qxT, sxT = oracle.quant_cols_T(x)
    oracle.dgrad(qd, sd, qw, sw)
    oracle.wgrad(qdT, sdT, qxT, sxT)
    qxd, sxd = oracle.quant_rows(xd)
    qwd, swd = oracle.quant_blocks(wd)
    oracle.fprop(qxd, sxd, qwd, swd)
    dt = time.perf_counter() - t0
    flops = 3 * gemm_flops(tokens, H, H) + gemm_flops(MD, F // 8, H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": (f"the full step's ops on a {tokens}-token slice (fold + 128x128 quantize of "
                       f"the full 4096x4096 W, 1x128/128x1 quantizers of X and dY[:{tokens}], "
                       f"FProp/DGrad/WGrad over {tokens} tokens, decode FProp 64 x {F // 8} x {H} "
                       f"incl. quantizing that weight slice); value = the slice's GEMM flops / "
                       f"oracle wall time")}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    step_ms, wall, per_op, dom, dom_ms, upd, normq, int8, w4, dec8, dec32 = run_gpu(args)
    table = op_table()
    kernels = {}
    for name, ms in per_op.items():
        bound, work = table[name]
        if bound == "mfma":
            ach = work / (ms * 1e-3) / 1e12
            kernels[name] = {"us": round(ms * 1e3, 2), "bound": "mfma", "achieved": round(ach, 1),
                             "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4)}
        else:
            ach = work / (ms * 1e-3) / 1e9
            kernels[name] = {"us": round(ms * 1e3, 2), "bound": "hbm", "achieved": round(ach, 1),
                             "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    gemm_total = 3 * gemm_flops(T, H, H) + decode_flops()
    value = gemm_total / (step_ms * 1e-3) / 1e12
    # the dominant kernel's roofline point: its launches inside the timed region
    bound, work = table[dom]
    peak = PEAK_FP8_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
    ach = work / (dom_ms * 1e-3) / (1e12 if bound == "mfma" else 1e9)
    roof = {"kernel": dom, "bound": bound, "achieved": round(ach, 1), "peak": peak,
            "unit": kernels[dom]["unit"], "frac": round(ach / peak, 4),
            "avg_launch_us": round(dom_ms * 1e3, 2), "traffic": measured_traffic(dom)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic (seeded; 8B-layer shapes)",
        "config": {"workload": ("8B-layer FP8 step: UAQ fold + 128x128 W quantize (4096x4096), "
                                "1x128 + 128x1 X quantize in one read (the 128x1 codes kept "
                                "for WGrad) + FProp 8192x4096x4096, fused dual dY "
                                "quantize-transpose, DGrad and WGrad (8192 tokens), decode "
                                "FProp 64x14336x4096"),
                   "tokens": T, "hidden": H, "decode_batch": MD, "decode_ffn": F,
                   "gemm_gflop_per_step": round(gemm_total / 1e9, 2)},
        "roofline": roof,
        "kernels": kernels,
        "weight_update": upd,
        "decode_8b": dec8,
        "decode_32b": dec32,
        "norm_quant": normq,
        "int8_w8a8": int8,
        "w4a16": w4,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = run_cpu_baseline(args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
