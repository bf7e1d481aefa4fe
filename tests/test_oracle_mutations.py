"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies the oracle and the CPU pin tests into a scratch directory, plants one slip in
the copy of oracle/rmsq_oracle.c -- the kind a reading of the pages or a typo could introduce --
and runs the pins there: every mutant must make at least one pin fail.  An unmutated copy must
pass, so a failure is the pins' doing and not the harness's.  The repository's oracle is never
modified.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle_pins.py", "test_oracle_formats.py", "test_oracle_act.py",
             "test_oracle_f16.py", "test_oracle_pad.py", "test_oracle_rope.py",
             "test_oracle_fp4_dynamic.py"]

# (name, text in rmsq_oracle.c, replacement, which occurrence (0 = first))
MUTANTS = [
    ("eps outside the root",
     "sqrt(ss / (double)n + (double)eps));", "sqrt(ss / (double)n) + (double)eps);", 0),
    ("mean of squares over n - 1",
     "sqrt(ss / (double)n + (double)eps));", "sqrt(ss / (double)(n - 1) + (double)eps));", 0),
    ("residual subtracted",
     "in16_to_f32(x[i], f16) + in16_to_f32(r[i], f16)",
     "in16_to_f32(x[i], f16) - in16_to_f32(r[i], f16)", 0),
    ("weight read backwards", "y[i] = t * in16_to_f32(w[i], f16);",
     "y[i] = t * in16_to_f32(w[n - 1 - i], f16);", 0),
    ("e4m3 ties to the odd code", "(d == bestd && (k & 1) == 0)", "(d == bestd && (k & 1) == 1)",
     0),
    ("e2m1 ties to the odd code", "(d == bestd && (k & 1) == 0)", "(d == bestd && (k & 1) == 1)",
     1),
    ("bf16 ties away from even", "else pick = (lo & 1u) ? hi : lo;", "else pick = hi;", 0),
    ("binary16 subnormal exponent", "mag = ldexp((double)m, -24);", "mag = ldexp((double)m, -25);",
     0),
    ("447 for the FP8 maximum", "float s = a / 448.0f;", "float s = a / 447.0f;", 0),
    ("E8M0 rounds up past an exact power of two", "if (ldexp(1.0, k) >= (double)s) return k;",
     "if (ldexp(1.0, k) > (double)s) return k;", 0),
    ("FP4 block scale over 4", "orc_e4m3_encode((a * gs) / 6.0f)",
     "orc_e4m3_encode((a * gs) / 4.0f)", 0),
    ("FP4 nibbles swapped", "(uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4))",
     "(uint8_t)(codes[2 * k + 1] | (codes[2 * k] << 4))", 0),
    ("column-major scale index transposed", "g * scale_ld + t : t * ng + g",
     "t * scale_ld + g : t * ng + g", 0),
    ("static scale used as a multiplier", "float r = 1.0f / scale;", "float r = scale;", 0),
    ("rotation sign", "*out_a = ac - bs;", "*out_a = ac + bs;", 0),
    ("NeoX pairs off by one", "ib = neox ? i + D / 2 : 2 * i + 1;",
     "ib = neox ? (i + D / 2 + 1) % D : 2 * i + 1;", 0),
    ("SiLU sign", "(1.0 + exp(-gd))", "(1.0 + exp(gd))", 0),
    ("batch FP4 scale without the e2m1 maximum", "(448.0f * 6.0f) / amax", "448.0f / amax", 0),
    ("zero element times an infinite multiplier", "return (y == 0.0f) ? y : y * mul;",
     "return y * mul;", 0),
    ("FP4 elements truncated toward zero", "codes[i] = orc_e2m1_encode(v);",
     "codes[i] = orc_e2m1_encode(truncf(v * 2.0f) * 0.5f);", 0),
    ("padding repeats the row's last value", "i < H ? f32_to_in16(y[i], f16) : 0",
     "i < H ? f32_to_in16(y[i], f16) : f32_to_in16(y[H - 1], f16)", 0),
    ("E8M0 byte biased by 128", "*e8m0_byte = k + 127;", "*e8m0_byte = k + 128;", 0),
    ("FP4 block whose scale underflows still divided", "if (d > 0.0f) {", "if (d >= 0.0f) {", 0),
    ("all-zero batch leaves an infinite global scale", "return (gs <= FLT_MAX) ? gs : FLT_MAX;",
     "return gs;", 0),
    ("new residual copied from x", "memcpy(residual_out + t * H, h, (size_t)H * sizeof(uint16_t));",
     "memcpy(residual_out + t * H, x + t * H, (size_t)H * sizeof(uint16_t));", 0),
    ("RoPE frequencies with exponent -i/D", "pow(base, -2.0 * (double)i / (double)D)",
     "pow(base, -1.0 * (double)i / (double)D)", 0),
    ("SiLU applied to the up half", "in16_to_f32(x[i], f16), (double)in16_to_f32(x[I + i], f16)",
     "in16_to_f32(x[I + i], f16), (double)in16_to_f32(x[i], f16)", 0),
]


def _replace_nth(text, old, new, nth):
    at = -1
    for _ in range(nth + 1):
        at = text.index(old, at + 1)
    return text[:at] + new + text[at + len(old):]


def _run_pins(tag, mutation):
    """Copy, mutate, run the pins; returns (tag, pytest exit status, last output line)."""
    import tempfile

    work = tempfile.mkdtemp(prefix="orc_mut_")
    try:
        ignore = shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__", "*.o")
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(work, "oracle"), ignore=ignore)
        os.makedirs(os.path.join(work, "tests"))
        for f in ["__init__.py", "conftest.py"] + PIN_FILES:
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(work, "tests", f))
        shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(work, "tests", "golden"))
        shutil.copytree(os.path.join(ROOT, "rmsnorm_quantization_amd"),
                        os.path.join(work, "rmsnorm_quantization_amd"), ignore=ignore)
        if mutation is not None:
            src = os.path.join(work, "oracle", "rmsq_oracle.c")
            text = open(src).read()
            old, new, nth = mutation
            open(src, "w").write(_replace_nth(text, old, new, nth))
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            *[os.path.join("tests", f) for f in PIN_FILES]],
                           cwd=work, capture_output=True, text=True, timeout=600)
        lines = (r.stdout + r.stderr).strip().splitlines()
        return tag, r.returncode, lines[-1] if lines else ""
    finally:
        shutil.rmtree(work, ignore_errors=True)


def test_every_planted_mistake_fails_a_pin():
    for name, old, _, nth in MUTANTS:  # every pattern is present (the mutant is real)
        _replace_nth(open(os.path.join(ROOT, "oracle", "rmsq_oracle.c")).read(), old, old, nth)
    jobs = [("unmutated", None)] + [(n, (o, w, k)) for n, o, w, k in MUTANTS]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _run_pins(*j), jobs))
    control = results[0]
    assert control[1] == 0, f"the unmutated copy fails its pins: {control[2]}"
    survivors = [(tag, last) for tag, rc, last in results[1:] if rc == 0]
    assert not survivors, f"mutants no pin catches: {survivors}"
    for tag, rc, last in results[1:]:
        assert rc == 1, f"{tag}: pytest exit {rc} ({last})"  # failed tests, not a crash
