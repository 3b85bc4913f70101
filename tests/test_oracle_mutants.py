"""The oracle's pins catch plausible mistakes: each case below plants one mistake in a copy of
the oracle source (a wrong rounding rule, a dropped saturation, a lost sign of zero, a
transposed or shifted scale index, a wrong constant, a reciprocal in place of the division, a
dropped absolute value, a double rounding, an off-by-one group, a wrong mean, a dropped eps
or gain in the norm, INT8 ties away from zero, a wrong INT8 divisor or scale index, an E2M1 tie to the odd code,
a wrong FP4 tensor divisor, a dropped FP4 block scale, 128x128 block codes formed with the
amax, half the scale or a per-element scale instead of the block scale) and runs the pin suite on that
copy, which must fail.  CPU only: the copies live in a temporary directory and the HIP library
is not involved."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "ties_away": ("double n = rint(ldexp(a, 3 - e));", "double n = round(ldexp(a, 3 - e));"),
    "no_saturation": ("if (a >= E4M3_MAX)\n        return sign | 0x7E;",
                      "if (a >= 1e30)\n        return sign | 0x7E;"),
    "sign_of_zero": ("uint8_t sign = signbit(v) ? 0x80 : 0x00;",
                     "uint8_t sign = v < 0 ? 0x80 : 0x00;"),
    "block_index_T": ("s[(r / GROUP) * nbj + c / GROUP]", "s[(c / GROUP) * nbj + r / GROUP]"),
    "scale_446": ("return amax / 448.0f;", "return amax / 446.0f;"),
    "reciprocal": ("float v = x / s;", "float v = x * (1.0f / s);"),
    "row_scale_shift": ("(double)s[r * ng + c / GROUP]", "(double)s[r * ng + (c + 1) / GROUP]"),
    "abs_sum": ("\n                a += fabs(p);", "\n                a += p;"),
    "abs_sum_sampled": ("\n            a += fabs(p);", "\n            a += p;"),
    "uaq_f32_quotient": ("double q = (double)orc_bf16_to_f32(w[r * ld + c]) / (double)s[c];",
                         "double q = (double)(orc_bf16_to_f32(w[r * ld + c]) / s[c]);"),
    "rms_mean_over_cols_plus_1": ("ss / (double)cols + (double)eps", "ss / (double)(cols + 1) + (double)eps"),
    "rms_no_eps": ("ss / (double)cols + (double)eps", "ss / (double)cols"),
    "rms_no_gain": ("* (double)gain[c] * inv", "* inv"),
    "int8_ties_away": ("double n = rint((double)v);", "double n = round((double)v);"),
    "int8_scale_128": ("float sc = amax / 127.0f;", "float sc = amax / 128.0f;"),
    "int8_gemm_scale_index": ("(double)sa[m] * (double)sb[n] * (double)acc",
                              "(double)sa[m] * (double)sb[m] * (double)acc"),
    "e2m1_ties_odd": ("if (dc < db || (dc == db && (c & 1) == 0))",
                      "if (dc < db || (dc == db && (c & 1) == 1))"),
    "nvfp4_tensor_divisor": ("float t = amax / 2688.0f;", "float t = amax / 2048.0f;"),
    "w4a16_no_block_scale": ("double w = orc_e2m1_decode(c) * orc_e4m3_decode(bscale[n * (K / 16) + kk / 16]);",
                             "double w = orc_e2m1_decode(c);"),
    "block_codes_divide_by_amax": (
        "q[r * k + c] = orc_quantize_value(orc_bf16_to_f32(w[r * ld + c]), sc);",
        "q[r * k + c] = orc_quantize_value(orc_bf16_to_f32(w[r * ld + c]), amax);"),
    "block_codes_half_scale": (
        "q[r * k + c] = orc_quantize_value(orc_bf16_to_f32(w[r * ld + c]), sc);",
        "q[r * k + c] = orc_quantize_value(orc_bf16_to_f32(w[r * ld + c]), sc * 0.5f);"),
    "block_codes_element_scale": (
        "q[r * k + c] = orc_quantize_value(orc_bf16_to_f32(w[r * ld + c]), sc);",
        "q[r * k + c] = orc_quantize_value(orc_bf16_to_f32(w[r * ld + c]), "
        "orc_group_scale(fabsf(orc_bf16_to_f32(w[r * ld + c]))));"),
    "column_group_short": ("int64_t r0 = g * GROUP, r1 = r0 + GROUP < rows ? r0 + GROUP : rows;",
                           "int64_t r0 = g * GROUP, r1 = r0 + GROUP - 1 < rows ? "
                           "r0 + GROUP - 1 : rows;"),
}


def _run_mutant(tmp_root, name, old, new):
    d = os.path.join(tmp_root, name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "*.tmp", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(d, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "quotient_check", "fold_check"))
    shutil.copy(os.path.join(ROOT, "qr_synth.py"), d)
    src_path = os.path.join(d, "oracle", "qr_oracle.c")
    src = open(src_path).read()
    with open(src_path, "w") as f:
        f.write(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=d, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, (r.stdout.strip().splitlines() or [""])[-1]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "qr_oracle.c")).read()
    for name, (old, _) in MUTANTS.items():
        assert src.count(old) == 1, f"mutant {name}: the original text is not unique in the oracle"
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run_mutant, str(tmp_path), name, old, new)
                for name, (old, new) in MUTANTS.items()}
        results = {name: f.result() for name, f in futs.items()}
    survived = {n: last for n, (rc, last) in results.items() if rc == 0}
    assert not survived, f"mistakes no pin catches: {survived}"
    # a failing run must be a failing pin, not a broken copy
    broken = {n: last for n, (rc, last) in results.items() if "failed" not in last}
    assert not broken, f"mutant runs that did not fail a test: {broken}"
