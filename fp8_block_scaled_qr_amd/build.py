"""Build the gfx950 library fp8_block_scaled_qr_amd/libqr.so from csrc/ with hipcc.

Always recompiles.  Object files go to _build/ at the repository root (not committed); the
shared library lands next to this file, where the Python binding loads it.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqr.so")
# the benchmark's streaming-read yardstick, a library of its own (not part of the qr ABI)
CEILING_SRC = "ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libqr_ceiling.so")

ARCH = "gfx950"
SOURCES = ["api.cpp", "quant.hip", "gemm.hip", "fp4.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall",
          # packed fp32 VALU ops stay off (plain fp32 code only)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep MFMA results in VGPRs: the promotion FMAs read them directly
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libqr.so")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [CEILING_SRC]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
