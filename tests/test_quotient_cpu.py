"""The GPU kernels' per-element arithmetic replayed on the host: the quantizers' quotient for
every (bf16 amax, bf16 x) pair (quotient_check.c) and the UAQ fold's rounding
(fold_check.c).  CPU only."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.mark.parametrize("divisor", ["448", "127"])
def test_quotient_matches_ieee_division_for_every_bf16_pair(tmp_path, divisor):
    """FP8 scales s = RN32(amax / 448) and INT8 scales s = RN32(amax / 127)."""
    exe = str(tmp_path / "quotient_check")
    cmd = ["gcc", "-O0", "-ffp-contract=off", "-fopenmp", os.path.join(HERE, "quotient_check.c"),
           "-o", exe, "-lm"]
    if _has_fma():
        cmd.insert(3, "-mfma")
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe, divisor], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    words = r.stdout.split()
    fields = dict(zip(words[2::2], map(int, words[3::2])))
    assert words[:2] == ["divisor", divisor]
    assert fields["pairs"] == 1065402240          # every finite (amax, x) with |x| <= amax
    assert fields["mismatches"] == 0, r.stdout
    assert r.returncode == 0


def test_fold_rounding_matches_exact_division(tmp_path):
    """The UAQ fold's two per-element routes (binary32 bracket plus one FMA sign test, and the
    binary64 fallback) against an exact integer RN_bf16(w / s) (see fold_check.c)."""
    exe = str(tmp_path / "fold_check")
    cmd = ["gcc", "-O1", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           os.path.join(HERE, "fold_check.c"), "-o", exe, "-lm"]
    if _has_fma():
        cmd.insert(3, "-mfma")
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    fields = dict(zip(r.stdout.split()[0::2], map(int, r.stdout.split()[1::2])))
    assert fields["pairs"] > 5 * 10**8
    assert fields["mismatches"] == 0, r.stdout
    assert fields["fast"] > fields["pairs"] // 2         # the binary32 route is the common one
    assert fields["close"] > 10**6                      # and is exercised near midpoints
    assert r.returncode == 0
