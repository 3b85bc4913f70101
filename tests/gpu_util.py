"""Helpers for the GPU parity tests: device transfer of the seeded inputs and the tolerance
check of the GEMMs against the oracle (test code only)."""
import numpy as np
import torch

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
                      bf16_out: bool = False):
    """Element-wise |gpu - Y| <= GEMM_TOL * S against the unrounded fp64 oracle Y.

    The tolerance covers the fp32 accumulation.  A bf16 output adds one more rounding of that
    fp32 value y (nearest even, at most 2^-8 |y| with |y| <= |Y| + GEMM_TOL * S), which on its
    own can exceed GEMM_TOL * S wherever |Y| / S > ~0.5; for bf16 outputs that rounding is
    added to the bound.  Returns (max err/S, max |Y|/S)."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == Y.shape == S.shape, (what, gpu.shape, Y.shape)
    assert np.all(np.isfinite(gpu)), what
    err = np.abs(gpu - Y)
    lim = GEMM_TOL * S
    if bf16_out:
        lim = lim + 2.0 ** -8 * (np.abs(Y) + GEMM_TOL * S)
    bad = np.flatnonzero(err.ravel() > lim.ravel())
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(S > 0, err / S, np.where(err > 0, np.inf, 0.0))
        ys = np.where(S > 0, np.abs(Y) / S, 0.0)
    assert bad.size == 0, (f"{what}: {bad.size} of {gpu.size} outside tolerance; worst err/S "
                           f"{rel.max():.3e} at {np.unravel_index(np.argmax(rel), rel.shape)}")
    return float(rel.max()) if rel.size else 0.0, float(ys.max()) if ys.size else 0.0


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
