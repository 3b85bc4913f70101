"""The oracle and the library's host side under AddressSanitizer + UndefinedBehaviorSanitizer
(CPU only).  Each test builds an instrumented copy in a temporary directory and runs an existing
CPU suite against it in a subprocess with the matching sanitizer runtime preloaded (Python itself
is not instrumented): the oracle pins against a gcc -fsanitize=address,undefined build of the
oracle, and the C-ABI validation tests against libqr.so with its host code instrumented (the GPU
code is built as usual; no kernel is launched).  Any sanitizer report aborts the subprocess and
fails the test.  Skipped when the compiler or the runtime is missing."""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_suite(suite, env_extra, preload):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", suite)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    tail = "\n".join((r.stdout + r.stderr).strip().splitlines()[-25:])
    assert r.returncode == 0, f"{suite} under the sanitizers:\n{tail}"
    assert " passed" in r.stdout, tail


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    rt = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc's ASan runtime not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([gcc, "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-shared", "-fPIC",
                    os.path.join(ROOT, "oracle", "qr_oracle.c"), "-o", lib, "-lm"], check=True)
    _run_suite("test_oracle_pins.py", {"QR_TEST_ORACLE_LIB": lib}, rt)


def test_abi_host_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from fp8_block_scaled_qr_amd import build as b
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang's ASan runtime not available")
    # host-side instrumentation only: every sanitizer flag goes to the host compilation
    san = ["-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        subprocess.run([hipcc] + b.COMMON + san + ["-c", os.path.join(b.CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(b.SOURCES)) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    lib = str(tmp_path / "libqr_san.so")
    subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={b.ARCH}", "-Xarch_host",
                    "-shared-libasan"] + san + objs + ["-o", lib], check=True, capture_output=True)
    _run_suite("test_abi_cpu.py", {"QR_TEST_LIB": lib}, rts[-1])
