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
  norm_quant_dec  the norm in front of the decode linear with its 1x128 quantize fused in:
                  h [64, 4096] -> codes and scales of RMSNorm(h) * gain
  fprop_decode    Y = X W^T            64 x 14336 x 4096 on the pre-quantized weight, bf16 out

After the warm-up, a breakdown pass of K steps brackets every launch with HIP events on the
stream it runs on (each op's time and roofline fraction).  The timed pass of K steps then
records events only around the dominant kernel's launch, so the step time carries no per-op
event overhead.  The JSON line reports the step's GEMM throughput (all GEMM flops / step
time) as `value`, each op's time with its roofline fraction, the roofline of the dominant
kernel from its launches in the timed pass, and the CPU oracle timed on bounded slices of the
same step (all cores and one core; quantizers and GEMMs separately).  Outside the step it also
times, each after a cache-evicting read where the op is HBM-bound:
  prefill_8b      the 1x128 quantize of X and FProp as one unit (combined TFLOP/s)
  tiny_fprop      the tiny FProp workload's three launches (microseconds only), as the host
                  issues them and with each call queued behind a long read (GPU-side time)
  decode_32b      the 32B decoder layer's four linears at decode batch 256 on the seeded,
                  UAQ-folded inputs of that workload
  ceilings        the best single-launch streaming rate over the decode GEMM's 60.84 MB
  weight_update   the batched re-quantization of a 32B layer's four weights (once per
                  optimizer step)
  norm_quant      the norm with the activation quantize fused in (FProp's operand producer)
  norm_quant_dual the norm emitting the 1x128 rows and the 128x1 columns from one read of h
  decode_8b       the 8B decoder layer's four FP8 linears at decode batch 64
  int8_w8a8, w4a16  the INT8 and 4-bit weight variants at the same shapes
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
        # the decode hidden state's norm with the 1x128 quantize fused in: read h and the gain,
        # write codes and scales
        "norm_quant_dec": ("hbm", MD * H * 2 + H * 4 + MD * H + MD * (H // g) * 4),
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
            ("norm_quant_dec", lambda: qr.qr_rmsnorm_quant_1x128(self.Xd, MD, H, H, self.gain, 1e-6,
                                                                 None, self.qXd, self.sXd)),
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
    extra = {}
    extra["prefill_8b"] = run_prefill_combined(torch, qr, st)
    extra["norm_quant"] = run_norm_quant(torch, qr, st)
    extra["norm_quant_dual"] = run_norm_quant_dual(torch, qr, st)
    extra["int8_w8a8"] = run_int8(torch, qr, st)
    extra["w4a16"] = run_w4a16(torch, qr, st)
    del st, ops
    torch.cuda.empty_cache()
    extra["tiny_fprop"] = run_tiny_fprop(torch, qr)
    extra["ceilings"] = run_ceilings(torch)
    torch.cuda.empty_cache()
    extra["decode_8b"] = run_decode_8b(torch, qr)
    torch.cuda.empty_cache()
    extra["weight_update"] = run_weight_update(torch, qr)
    torch.cuda.empty_cache()
    extra["decode_32b"] = run_decode_32b(torch, qr)
    torch.cuda.empty_cache()
    return step_ms, wall, per_op, dom, dom_ms, extra


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


def run_norm_quant_dual(torch, qr, st, iters=20):
    """The norm emitting both activation layouts on the prefill hidden state [8192, 4096] (the
    step's X stands in for h; the gain carries the UAQ s): the row statistics, then the 1x128
    rows for FProp and the 128x1 columns (transposed) for WGrad from one read of h.  Algorithmic
    bytes: h once, the gain, both codes and scales, inv_rms."""
    dev = "cuda:0"
    g = st.s.clone()
    inv = torch.empty(T, dtype=torch.float32, device=dev)
    q, qT = torch.empty((T, H), dtype=torch.uint8, device=dev), torch.empty((H, T), dtype=torch.uint8, device=dev)
    s = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    sT = torch.empty((H, T // 128), dtype=torch.float32, device=dev)
    f = lambda: qr.qr_rmsnorm_quant_dual(st.X, T, H, H, g, 1e-6, inv, None, q, s, qT, sT)
    us = _median_us(torch, f, iters)
    nbytes = T * H * 2 + H * 4 + 2 * T * H + 2 * T * (H // 128) * 4 + T * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "RMSNorm (gain carrying the UAQ s) of h [8192, 4096] with its 1x128 rows "
                        "and 128x1 columns (transposed) quantized from one read of h, inv_rms out "
                        "(two launches: row statistics, then the tiles)",
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
    del ws, items
    torch.cuda.empty_cache()
    upd = {"workload": "32B decoder layer weights (QKV 7168x5120, O 5120x5120, gate+up "
                       "55296x5120, down 5120x27648) re-quantized 128x128 with transposed "
                       "copies, one batched call",
           "us": round(us, 1), "bound": "hbm", "bytes": nbytes, "achieved": round(gbs, 1),
           "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "launches": 1}
    return upd


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


def run_decode_32b(torch, qr, iters=20):
    """The 32B decoder layer's four linears at decode batch 256 on the seeded, UAQ-folded
    inputs of that workload (qr_synth.decode_32b_set: W ~ N(0, 0.02), s ~ U(1.5, 4) per input
    column, X = s (.) X0 with 1% outlier channels): W' = fold(W, s) and its 128x128 codes (one
    call, untimed: a one-time preprocessing), X's 1x128 codes (untimed: the norm in front
    produces them), then FProp with bf16 out, timed after a cache-evicting read so the weight
    streams from HBM.  Algorithmic bytes = weight codes + block scales + activation codes and
    scales + bf16 Y."""
    import qr_synth
    dev = "cuda:0"
    M, g = 256, 128
    out, tot_us, tot_fl, tot_b = {}, 0.0, 0.0, 0
    t0 = time.time()
    for lin in qr_synth.decode_32b_set():
        name = lin.name.replace("decode_32b_", "")
        n, k = lin.N, lin.K
        w = torch.from_numpy(lin.w().view(np.int16)).to(dev).view(torch.bfloat16)
        sc = torch.from_numpy(lin.uaq_s()).to(dev)
        q = torch.empty((n, k), dtype=torch.uint8, device=dev)
        s = torch.empty((n // g, k // g), dtype=torch.float32, device=dev)
        qr.qr_uaq_fold_quant_w_128x128(w, n, k, k, sc, w, None, q, s)   # in place
        del w
        x = torch.from_numpy(lin.x().view(np.int16)).to(dev).view(torch.bfloat16)
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
                     "frac_mfma": round(tf / PEAK_FP8_TFLOPS, 4),
                     "k_splits": nb // (M * n * 4) if nb else 1}
        tot_us, tot_fl, tot_b = tot_us + us, tot_fl + fl, tot_b + by
        del q, s, sc, x, qx, sx, y, ws
        torch.cuda.empty_cache()
    log(f"decode_32b inputs drawn and timed in {time.time() - t0:.1f}s")
    out["layer"] = {"us": round(tot_us, 1), "tflops": round(tot_fl / (tot_us * 1e-6) / 1e12, 1),
                    "gbs": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
                    "frac_hbm": round(tot_b / (tot_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "frac_mfma": round(tot_fl / (tot_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
                    "bytes": tot_b, "gflop": round(tot_fl / 1e9, 2)}
    out["workload"] = ("32B decoder layer at decode batch 256: QKV 5120->7168, O 5120->5120, "
                       "gate+up 5120->55296, down 27648->5120; seeded UAQ-folded weights "
                       "(s ~ U(1.5, 4)) and activations s (.) X0, FProp, bf16 out, each after a "
                       "cache-evicting read")
    return out


def run_tiny_fprop(torch, qr, iters=50):
    """The tiny FProp workload (X [256, 512] with 4 outlier channels, W [512, 512], fp32 out):
    the 1x128 quantize of X, the 128x128 quantize of W and the GEMM, launched back to back; a
    launch-latency-bound case, reported in microseconds only."""
    import qr_synth
    dev = "cuda:0"
    lin = qr_synth.tiny_fprop()
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    x, w = bf(lin.x()), bf(lin.w())
    M, N, K = lin.M, lin.N, lin.K
    qx, sx = torch.empty((M, K), dtype=torch.uint8, device=dev), torch.empty((M, K // 128), device=dev)
    qw, sw = torch.empty((N, K), dtype=torch.uint8, device=dev), torch.empty((N // 128, K // 128), device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    nb = qr.qr_gemm_workspace_bytes(qr.QR_GEMM_FPROP, M, N, K)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    parts = {
        "quant_x": lambda: qr.qr_quant_act_1x128(x, M, K, K, qx, sx, None, None),
        "quant_w": lambda: qr.qr_quant_w_128x128(w, N, K, K, qw, sw, None, None),
        "gemm": lambda: qr.qr_gemm_fp8_bsfprop(qx, sx, qw, sw, M, N, K, y, qr.QR_OUT_F32, ws, nb),
    }
    out = {k: round(_median_us(torch, f, iters, flush=False), 2) for k, f in parts.items()}

    def whole():
        for f in parts.values():
            f()
    out["total_us"] = round(_median_us(torch, whole, iters, flush=False), 2)
    # The same calls with a long read queued ahead of each, so every launch is already in the
    # queue when the GPU reaches it: the GPU-side time, dispatch gaps included. The figures
    # above are paced by the host's per-call cost (the GPU waits for each launch).
    for k, f in list(parts.items()) + [("total", whole)]:
        out[f"queued_{k}_us"] = round(_median_us(torch, f, iters, flush=True), 2)
    out["workload"] = "tiny FProp: X [256, 512] 1x128 + W [512, 512] 128x128 quantize, GEMM to fp32 [256, 512]"
    return out


def run_prefill_combined(torch, qr, st, iters=20):
    """The prefill FProp with its activation quantize in front, as one unit: the 1x128 quantize
    of X [8192, 4096] (rows only) and the GEMM 8192x4096x4096 (bf16 out), each after a
    cache-evicting read, and the pair back to back after one."""
    dev = "cuda:0"
    q = torch.empty((T, H), dtype=torch.uint8, device=dev)
    s = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    ws, nb = st.ws["fprop"]
    quant = lambda: qr.qr_quant_act_1x128(st.X, T, H, H, q, s, None, None)
    gemm = lambda: qr.qr_gemm_fp8_bsfprop(q, s, st.qW, st.sW, T, H, H, st.Y, qr.QR_OUT_BF16, ws, nb)

    def both():
        quant()
        gemm()
    qu, gu, bu = (_median_us(torch, f, iters) for f in (quant, gemm, both))
    qb = T * H * 3 + T * (H // 128) * 4
    fl = gemm_flops(T, H, H)
    return {"workload": "1x128 quantize of X [8192, 4096] then FProp 8192x4096x4096, bf16 out",
            "quant_us": round(qu, 2), "quant_gbs": round(qb / qu / 1e3, 1),
            "quant_frac_hbm": round(qb / qu / 1e3 / PEAK_HBM_GBS, 4),
            "gemm_us": round(gu, 2), "gemm_tflops": round(fl / gu / 1e6, 1),
            "combined_us": round(bu, 2), "combined_tflops": round(fl / bu / 1e6, 1),
            "combined_frac_mfma": round(fl / bu / 1e6 / PEAK_FP8_TFLOPS, 4)}


def run_ceilings(torch, iters=20):
    """What one launch streaming the decode GEMM's 60.84 MB (64 x 14336 x 4096: weight codes and
    scales, activation, output) can reach on this GPU: a plain contiguous read of that many
    bytes (libqr_ceiling.so; 256-thread workgroups, each reading one contiguous share, 16 bytes
    per lane and four accesses in flight) over a sweep of grid sizes, after a cache-evicting
    read, best grid reported; torch's copy of the same bytes for comparison.  A yardstick for
    the decode kernel, not a roofline: the roofline stays the published 8 TB/s."""
    import ctypes
    import fp8_block_scaled_qr_amd as qr
    from fp8_block_scaled_qr_amd import build as qb
    dev = "cuda:0"
    nbytes = F * H + (F // 128) * (H // 128) * 4 + MD * H + MD * (H // 128) * 4 + MD * F * 2
    nbytes -= nbytes % 16
    lib = ctypes.CDLL(qb.CEILING_LIB)
    lib.qr_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p]
    lib.qr_ceiling_stream_read.restype = ctypes.c_int
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sweep = {}
    for grid in (256, 512, 1024, 2048, 4096, 8192, 16384):
        def f(grid=grid):
            rc = lib.qr_ceiling_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, grid,
                                            ctypes.c_void_p(sink.data_ptr()), stream)
            if rc != 0:
                raise RuntimeError(f"qr_ceiling_stream_read: {rc}")
        us = _median_us(torch, f, iters)
        sweep[grid] = {"us": round(us, 2), "gbs": round(nbytes / us / 1e3, 1)}
    best = min(sweep, key=lambda g: sweep[g]["us"])
    dst = torch.empty_like(buf)
    cu = _median_us(torch, lambda: dst.copy_(buf), iters)
    return {"workload": f"one contiguous read of {nbytes / 1e6:.2f} MB (the 64x14336x4096 decode "
                        f"GEMM's algorithmic bytes) after a cache-evicting read",
            "bytes": nbytes, "read_sweep": sweep, "best_grid": best,
            "best_us": sweep[best]["us"], "best_gbs": sweep[best]["gbs"],
            "best_frac_hbm": round(sweep[best]["gbs"] / PEAK_HBM_GBS, 4),
            "torch_copy": {"us": round(cu, 2), "gbs_read_plus_write": round(2 * nbytes / cu / 1e3, 1)}}


# ------------------------------------------------------------------ CPU oracle baseline

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_leg(oracle, x, dy, w, s, xd, wd, gemm_tokens):
    """One timing of the oracle on the step's operations: the quantizers (fold + 128x128 blocks
    with the transposed copy's work, X rows + columns, dY rows + columns, the decode activation)
    over the given slices, then the four GEMMs with their contraction or token dim cut to
    gemm_tokens (the decode one on the decode weight slice).  Returns (quant seconds, quant
    bytes, GEMM seconds, GEMM flops)."""
    t = x.shape[0]
    t0 = time.perf_counter()
    wf, _ = oracle.uaq_fold(w, s, np.ones(w.shape[1], np.float32))
    qw, sw = oracle.quant_blocks(wf)
    qx, sx = oracle.quant_rows(x)
    qxT, sxT = oracle.quant_cols_T(x)
    qd, sd = oracle.quant_rows(dy)
    qdT, sdT = oracle.quant_cols_T(dy)
    qxd, sxd = oracle.quant_rows(xd)
    qwd, swd = oracle.quant_blocks(wd)
    tq = time.perf_counter() - t0
    n, k = w.shape
    qbytes = (n * k * 2 * 2 + 2 * n * k                     # fold (read + write), codes
              + 2 * (t * k * 2 + 2 * t * k + 8 * t * k // 128)   # X and dY: read, both layouts
              + xd.size * 3 + wd.size * 3)                   # decode activation and weight slice
    g = gemm_tokens
    t0 = time.perf_counter()
    oracle.fprop(qx[:g], sx[:g], qw, sw)
    oracle.dgrad(qd[:g], sd[:g], qw, sw)
    oracle.wgrad(np.ascontiguousarray(qdT[:, :g]), np.ascontiguousarray(sdT[:, : g // 128]),
                 np.ascontiguousarray(qxT[:, :g]), np.ascontiguousarray(sxT[:, : g // 128]))
    oracle.fprop(qxd, sxd, qwd, swd)
    tg = time.perf_counter() - t0
    flops = 3 * gemm_flops(g, n, k) + gemm_flops(xd.shape[0], wd.shape[0], k)
    return tq, qbytes, tg, flops


def run_cpu_baseline(tokens_all=4096, tokens_one=128):
    """The oracle (plain C, fp64 products, OpenMP over rows) on bounded slices of the same
    step, timed twice: with every thread the OpenMP runtime has (all host cores) and with one.
    The all-core leg quantizes the first 2 * tokens_all tokens of X and dY and runs the GEMMs
    over tokens_all tokens; the one-core leg uses 8 * tokens_one and tokens_one.  Both fold and
    quantize the full 4096x4096 weight and a 1792-row slice of the decode weight."""
    import ctypes
    import oracle
    import qr_synth
    oracle.lib()
    gomp = ctypes.CDLL("libgomp.so.1")
    all_threads = int(gomp.omp_get_max_threads())
    s = qr_synth.uniform_f32(3011, H, 1.5, 4.0)
    x = qr_synth.normal_bf16(3001, (T, H), 1.0, 3003, qr_synth.n_outliers(H), col_scale=s)
    w = qr_synth.normal_bf16(3002, (H, H), 0.02)
    dy = qr_synth.backward_8b_dy()
    dec = qr_synth.decode_8b()
    xd, wd = dec.x(), dec.w()[: F // 8]
    legs = {}
    for name, threads, qtok, gtok in (("all_cores", all_threads, 2 * tokens_all, tokens_all),
                                      ("one_core", 1, 8 * tokens_one, tokens_one)):
        gomp.omp_set_num_threads(threads)
        tq, qb, tg, fl = _oracle_leg(oracle, np.ascontiguousarray(x[:qtok]),
                                     np.ascontiguousarray(dy[:qtok]), w, s, xd, wd, gtok)
        legs[name] = {"threads": threads,
                      "quantize": {"tokens": qtok, "seconds": round(tq, 3), "bytes": qb,
                                   "GB/s": round(qb / tq / 1e9, 3)},
                      "gemm": {"tokens": gtok, "seconds": round(tg, 3), "gflop": round(fl / 1e9, 2),
                               "GFLOP/s": round(fl / tg / 1e9, 3)}}
    gomp.omp_set_num_threads(all_threads)
    a = legs["all_cores"]
    return {"value": round(a["gemm"]["GFLOP/s"] / 1e3, 5), "unit": "TFLOP/s",
            "cores": all_threads, "kind": "oracle", "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count(),
            "sample": (f"the step's operations on bounded slices: quantizers (UAQ fold + 128x128 "
                       f"blocks of the full 4096x4096 W, 1x128 rows and 128x1 columns of X and "
                       f"dY, the decode activation and a {F // 8}x{H} decode-weight slice) and "
                       f"GEMMs (FProp, DGrad, WGrad over the token slice, decode FProp "
                       f"{MD}x{F // 8}x{H}); all cores: {2 * tokens_all} tokens quantized, "
                       f"{tokens_all} in the GEMMs; one core: {8 * tokens_one} and {tokens_one}; "
                       f"value = all-core GEMM flops / oracle seconds"),
            "legs": legs}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens in the all-core CPU oracle's GEMMs (twice that quantized)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    step_ms, wall, per_op, dom, dom_ms, extra = run_gpu(args)
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
        "wall_s": round(wall, 3),
    }
    out.update(extra)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = run_cpu_baseline(args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
