"""Mutation test of the oracle's pins (CPU only).

Each mutant plants one plausible mistake in a copy of oracle.c, built into a
temporary directory; the pin tests (test_oracle_gemm.py, test_oracle_logprob.py)
run against it in a subprocess and must fail.  The unmutated control, built the
same way, must pass.  The committed oracle source is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_gemm.py", "tests/test_oracle_logprob.py"]

MUTANTS = {
    "scale index shifted by one group": (
        "w[k] = (double)qr[k] * f16_as_double(sr[k / 32]);",
        "w[k] = (double)qr[k] * f16_as_double(sr[(k / 32 + 1) % G]);"),
    "neighbouring column mixed in": (
        "acc += w[k] * (double)bf16_as_float(xr[k]);",
        "acc += w[k] * (double)bf16_as_float((xr + (j ^ 1 < t ? (j ^ 1) - j : 0) * ldx)[k]);"),
    "absolute mass keeps the signs": (
        "a += fabs(w[k] * (double)bf16_as_float(xr[k]));", "a += w[k] * (double)bf16_as_float(xr[k]);"),
    "fp16 subnormal scales flushed": ("v = ldexp((double)m, -24);", "v = 0.0;"),
    "fp32 instead of fp64 accumulation": ("double acc = 0.0;", "float acc = 0.0f;"),
    "block fold reversed": (
        "S = (b == 0) ? P : S + P;",
        "S = (b == 0) ? P : S + P; (void)0;\n            }\n            { S = 0.0f; for (int64_t b = nb - 1; b >= 0; --b) {"
        " float P = tree_sum(e + b * block, block); S = (b == nb - 1) ? P : S + P; }"),
    "sequential in-block sum": (
        "    if (w == 1) return e[0];\n    float left",
        "    if (w >= 1) { float a = e[0]; for (int64_t i = 1; i < w; ++i) a += e[i]; return a; }\n    float left"),
    "strided in-block tree": (
        "    if (w == 1) return e[0];\n    float left",
        "    if (w > 1) { float *a = (float *)malloc((size_t)w * sizeof(float)); memcpy(a, e, (size_t)w * sizeof(float));"
        " for (int64_t h = w / 2; h >= 1; h /= 2) for (int64_t i = 0; i < h; ++i) a[i] = a[i] + a[i + h];"
        " float r = a[0]; free(a); return r; }\n    if (w == 1) return e[0];\n    float left"),
    "per-block max shift": (
        "float shifted = bf16_as_float(l[v]) - m;",
        "float bm = -INFINITY; for (int64_t u = (v / block) * block; u < (v / block + 1) * block && u < V; ++u) {"
        " float lu = bf16_as_float(l[u]); if (lu > bm) bm = lu; } float shifted = bf16_as_float(l[v]) - bm;"),
    "padding not exactly zero": ("e[v] = 0.0f;", "e[v] = 1e-30f;"),
    "positive-zero (direct) form": ("out[j] = -d;", "out[j] = st - Lg;"),
    "direct form with the blockwise sign": ("out[j] = st - Lg;", "out[j] = -(Lg - st);"),
    "argmax ties take the last index": ("if (isnan(lv) || lv > bv) {", "if (isnan(lv) || lv >= bv) {"),
    "argmax skips NaN": ("if (isnan(lv) || lv > bv) {", "if (lv > bv) {"),
    "bf16 rounding truncates": ("double r = nearbyint(a / ulp) * ulp;", "double r = floor(a / ulp) * ulp;"),
    "exp32 through fp32 libm": (
        "float oracle_exp32(float x) { return (float)expl((long double)x); }",
        "float oracle_exp32(float x) { return (float)(double)expf(x); }"),
}


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", *oracle.CFLAGS, str(c), "-o", str(so), "-lm"], check=True)
    return so


def _run_pins(so):
    env = dict(os.environ, W8INV_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode


def test_unmutated_control_passes(tmp_path):
    so = _build(open(SRC).read(), tmp_path, "control")
    assert _run_pins(so) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_killed(name, tmp_path):
    a, b = MUTANTS[name]
    src = open(SRC).read()
    assert a in src, f"mutation site for {name!r} not found"
    so = _build(src.replace(a, b, 1), tmp_path, "mutant")
    assert _run_pins(so) != 0, f"pins did not detect: {name}"
