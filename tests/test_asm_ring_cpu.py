"""Static check of the skinny-M GEMM's hand-counted load ring (CPU only: compiles the GEMM to
gfx950 assembly with the library's own flags and scans it).

The decode kernel issues its ring loads through inline asm so that the compiler adds no
waits of its own; in exchange the compiler does not know that those destination registers
are written late.  Correctness then rests on two facts this test checks in the generated
code of every instantiation: between a ring load and the s_waitcnt vmcnt that retires it
(loads retire in order), no instruction reads or writes the load's destination registers,
and no later load overwrites them.  The scan is linear over the code as emitted (it follows
fall-through paths, including the loop exit), which is where a register reuse after the last
refill would show."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "fp8_block_scaled_qr_amd"))


def _regs(text):
    out = set()
    for kind, lo, hi in re.findall(r"\b([va])\[(\d+):(\d+)\]", text):
        out |= {f"{kind}{i}" for i in range(int(lo), int(hi) + 1)}
    for kind, n in re.findall(r"\b([va])(\d+)\b", text):
        out.add(f"{kind}{n}")
    return out


def scan(lines):
    """Returns the list of hazards: (line index, instruction)."""
    pending = []   # [dest registers, number of VMEM loads issued after it]
    issues = []
    for i, line in enumerate(lines):
        op = line.split()[0]
        args = line[len(op):]
        if op == "s_waitcnt" and "vmcnt" in line:
            n = int(re.search(r"vmcnt\((\d+)\)", line).group(1))
            pending = [p for p in pending if p[1] < n]
            continue
        if line.endswith(":") or op.startswith(("s_cbranch", "s_branch")):
            continue
        parts = args.split(",")
        if op.startswith(("buffer_load", "global_load")):
            dst, srcs = _regs(parts[0]), _regs(",".join(parts[1:]))
            for regs, _ in pending:
                if regs & (srcs | dst):
                    issues.append((i, line))
            pending = [[r, n + 1] for r, n in pending]
            pending.append([dst, 0])
            continue
        if op.startswith("ds_write") or op.startswith(("buffer_store", "global_store")):
            used, written = _regs(args), set()
        else:
            used, written = _regs(",".join(parts[1:])), _regs(parts[0]) if parts else set()
        for regs, _ in pending:
            if regs & (used | written):
                issues.append((i, line))
    return issues


def kernel_bodies(asm, name_part):
    out = {}
    for m in re.finditer(r"^(_Z\S*" + name_part + r"\S*):", asm, re.M):
        body = asm[m.end():]
        body = body[:body.index("s_endpgm")]
        out[m.group(1)] = [l.strip() for l in body.split("\n")
                           if l.strip() and not l.strip().startswith((".", ";"))]
    return out


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    import build as B
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    cmd = [B.hipcc()] + B.COMMON + ["--cuda-device-only", "-S",
                                    os.path.join(B.CSRC, "gemm.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("hipcc unavailable: " + r.stderr[-300:])
    return open(out).read()


def test_skinny_ring_registers_untouched_until_waited(gemm_asm):
    bodies = kernel_bodies(gemm_asm, "k_gemm_skinny")
    assert len(bodies) >= 6, "expected the skinny instantiations (3 row-tile counts x 2 outputs)"
    for name, lines in bodies.items():
        assert any("buffer_load" in l for l in lines), name
        issues = scan(lines)
        assert not issues, (name, issues[:5])


def test_scan_detects_a_reused_register():
    """The scanner itself: a register written while its load is pending is reported, and a
    wait that retires the load clears it."""
    bad = ["buffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen",
           "buffer_load_dword v9, v2, s[0:3], 0 offen",
           "v_mov_b32_e32 v5, 0"]
    assert len(scan(bad)) == 1
    good = bad[:2] + ["s_waitcnt vmcnt(1)", "v_mov_b32_e32 v5, 0"]
    assert scan(good) == []
    early = bad[:2] + ["s_waitcnt vmcnt(1)", "v_add_u32_e32 v3, v9, v9"]
    assert len(scan(early)) == 1
