"""Seeded synthetic inputs for the FP8 quantize-and-multiply path.

The tests, the benchmark and the smoke check draw every input from here, and both the HIP
library and the reference oracle consume the same bytes.  This module holds none of the
method's arithmetic: it only draws normals and uniforms, multiplies chosen outlier channels,
and rounds float32 to bf16 (round-to-nearest-even) to produce the bf16 tensors that the
quantizers take as input.

Recipe (layer shapes of 8B- and 32B-parameter actors; the pages' real models and math-RL
datasets are not used and not needed):

* ``numpy.random.Generator(PCG64(seed))``; float64 standard normals times sigma -> float32
  -> bf16 (RNE).  Large tensors are drawn row-chunk by row-chunk from one generator, which
  yields the same stream as a single draw.
* Outlier channels: ``Generator(PCG64(idx_seed)).choice(K, round(0.01*K), replace=False)``
  (4 channels for the tiny case), multiplied by 20 in float32 before the bf16 rounding.
* UAQ scales: ``Generator(PCG64(seed)).uniform(1.5, 4.0, K)`` as float32 (per input column).
"""
from dataclasses import dataclass, field

import numpy as np

OUTLIER_MULT = 20.0


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def n_outliers(k: int) -> int:
    return int(round(0.01 * k))


def outlier_index(seed: int, k: int, n: int) -> np.ndarray:
    return np.sort(np.random.Generator(np.random.PCG64(seed)).choice(k, n, replace=False))


def normal_bf16(seed: int, shape, std: float, outlier_seed=None, n_out: int = 0,
                col_scale=None, chunk_rows: int = 2048) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws; optional outlier columns (x20) and an optional
    per-column float32 multiplier (the activation a norm with that gain would emit)."""
    rows, cols = shape
    g = np.random.Generator(np.random.PCG64(seed))
    idx = outlier_index(outlier_seed, cols, n_out) if n_out else None
    out = np.empty((rows, cols), np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        blk = (g.standard_normal((r1 - r0, cols)) * std).astype(np.float32)
        if idx is not None:
            blk[:, idx] *= np.float32(OUTLIER_MULT)
        if col_scale is not None:
            blk *= np.asarray(col_scale, np.float32)[None, :]
        out[r0:r1] = f32_to_bf16_bits(blk)
    return out


def uniform_f32(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed)).uniform(lo, hi, n).astype(np.float32)


# ---------------------------------------------------------------- workloads

@dataclass
class Linear:
    """One linear layer's synthetic tensors (bf16 bits as uint16 numpy arrays)."""
    name: str
    M: int
    N: int
    K: int
    x_seed: int
    w_seed: int
    idx_seed: int
    n_out: int
    x_std: float = 1.0
    w_std: float = 0.02
    s_seed: int = None          # UAQ per-input-column scale (None: no fold)
    _cache: dict = field(default_factory=dict, repr=False)

    def uaq_s(self):
        if self.s_seed is None:
            return None
        if "s" not in self._cache:
            self._cache["s"] = uniform_f32(self.s_seed, self.K, 1.5, 4.0)
        return self._cache["s"]

    def x(self):
        """Activation [M, K]: N(0,1) with outlier channels; with a UAQ scale s it is the
        output of a norm whose gain carries s, i.e. s (.) X0 per column."""
        return normal_bf16(self.x_seed, (self.M, self.K), self.x_std, self.idx_seed, self.n_out,
                           col_scale=self.uaq_s())

    def w(self):
        """Weight [N, K] (before any UAQ fold)."""
        return normal_bf16(self.w_seed, (self.N, self.K), self.w_std)


def tiny_fprop() -> Linear:
    """X [256, 512] N(0,1) with 4 outlier channels x20, W [512, 512] N(0, 0.02); fp32 out."""
    return Linear("tiny_fprop", 256, 512, 512, 1001, 1002, 1003, 4)


def decode_8b() -> Linear:
    """8B-shaped decode FProp: X [64, 4096] with 1% outlier channels, W [14336, 4096]."""
    return Linear("decode_8b", 64, 14336, 4096, 2001, 2002, 2003, n_outliers(4096))


def prefill_8b() -> Linear:
    """8B-shaped prefill/training FProp: X [8192, 4096] with 1% outliers, W [4096, 4096]."""
    return Linear("prefill_8b", 8192, 4096, 4096, 3001, 3002, 3003, n_outliers(4096))


def backward_8b_dy() -> np.ndarray:
    """Output gradient dY [8192, 4096] ~ N(0, 1e-3^2) for the prefill_8b layer."""
    return normal_bf16(4001, (8192, 4096), 1e-3)


def decode_32b_set():
    """32B-shaped decoder-layer linears at decode batch 256 with per-column UAQ scales
    s ~ U(1.5, 4): QKV 5120->7168, O 5120->5120, gate+up 5120->2x27648, down 27648->5120."""
    shapes = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 55296, 5120),
              ("down", 5120, 27648)]
    out = []
    for l, (name, n, k) in enumerate(shapes):
        out.append(Linear(f"decode_32b_{name}", 256, n, k, 5021 + l, 5001 + l, 5031 + l,
                          n_outliers(k), s_seed=5011 + l))
    return out
