"""Static check of the direct-to-LDS load helpers' use of M0 (CPU only: compiles the kernels that
use them to gfx950 assembly with the library's own flags and scans it).

`buffer_load_* ... lds` takes its LDS address from M0, so the helpers set M0 in the same
inline-asm statement as the load and name M0 as clobbered.  That is only sound while no
compiler-generated instruction relies on M0 across those statements.  This test checks it in
the generated code: every instruction that mentions M0 is the helpers' `s_mov_b32 m0, sN`, and
the next instruction is the direct-to-LDS load it addresses."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "fp8_block_scaled_qr_amd"))


def m0_issues(lines):
    """(index, instruction) of every M0 use that is not a helper's set-then-load pair."""
    issues = []
    for i, line in enumerate(lines):
        if not re.search(r"\bm0\b", line):
            continue
        ok = (re.fullmatch(r"s_mov_b32 m0, s\d+", line) is not None and i + 1 < len(lines)
              and lines[i + 1].startswith("buffer_load_") and lines[i + 1].endswith(" lds"))
        if not ok:
            issues.append((i, line))
    return issues


def instructions(asm):
    out = []
    for l in asm.split("\n"):
        l = l.split(";")[0].strip()
        if l and not l.startswith(".") and not l.endswith(":"):
            out.append(l)
    return out


@pytest.mark.parametrize("src", ["gemm.hip", "fp4.hip"])
def test_m0_only_set_for_the_lds_loads(src, tmp_path):
    import build as B
    out = str(tmp_path / (src + ".s"))
    cmd = [B.hipcc()] + B.COMMON + ["--cuda-device-only", "-S", os.path.join(B.CSRC, src),
                                    "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("hipcc unavailable: " + r.stderr[-300:])
    lines = instructions(open(out).read())
    lds_loads = [l for l in lines if l.startswith("buffer_load_") and l.endswith(" lds")]
    assert lds_loads, src
    issues = m0_issues(lines)
    assert not issues, issues[:5]
    # every direct-to-LDS load is addressed by the instruction right before it
    for i, l in enumerate(lines):
        if l.startswith("buffer_load_") and l.endswith(" lds"):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", lines[i - 1]), (i, lines[i - 1], l)


def test_scan_detects_other_m0_uses():
    good = ["s_mov_b32 m0, s4", "buffer_load_dwordx4 v1, s[0:3], 0 offen lds"]
    assert m0_issues(good) == []
    assert len(m0_issues(["s_mov_b32 m0, s4", "v_mov_b32_e32 v1, 0"])) == 1
    assert len(m0_issues(good + ["s_mov_b32 s5, m0"])) == 1
    assert len(m0_issues(["v_readlane_b32 s1, v1, m0"])) == 1
