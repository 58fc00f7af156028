"""The oracle pins must catch plausible mistakes in the oracle.

Each case copies ``oracle/qgemv_oracle.c``, plants one mistake by a text
substitution (a swapped nibble, a wrong index, a dropped term, a lost sign),
builds the copy with gcc on the CPU, and runs the pin suite against it through
``QGEMV_ORACLE_LIB``.  The suite must fail for every mutant and pass for the
unmodified source.  CPU only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qgemv_oracle.c")

MUTANTS = {
    "int4 nibble order": ("return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                          "return (k % 2 == 0) ? (byte >> 4) : (byte & 0x0F);"),
    "int4 zero-point nibble": ("return (b % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                               "return (b % 2 == 0) ? (byte >> 4) : (byte & 0x0F);"),
    "int4 block index": ("int64_t b = k / block_size;", "int64_t b = k / 32;"),
    "int4 zero point dropped": ("return s * (double)(q - z);", "return s * (double)q;"),
    "q4k scale high bits from wrong byte": ("*s = (sc[cc + 4] & 0x0F) | ((sc[cc - 4] >> 6) << 4);",
                                            "*s = (sc[cc + 4] & 0x0F) | ((sc[cc] >> 6) << 4);"),
    "q4k min low bits": ("*m = sc[cc + 4] & 63;", "*m = sc[cc] & 63;"),
    "q4k negation as subtraction": ("*mv = -(float)(dmin * (double)m);",
                                    "*mv = 0.0f - (float)(dmin * (double)m);"),
    "q4k quant nibble order": ("return (cc % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                               "return (cc % 2 == 0) ? (byte >> 4) : (byte & 0x0F);"),
    "q4k quant byte index": ("uint8_t byte = qs[32 * g + l];", "uint8_t byte = qs[16 * g + l];"),
    "plane row-major instead of chunk-major": ("plane[(c * N + n) * 2 + 0] = dv;",
                                               "plane[(n * nchunk + c) * 2 + 0] = dv;"),
    "f16 exponent bias": ("v = ldexp((double)(1024 + f), e - 25);",
                          "v = ldexp((double)(1024 + f), e - 24);"),
    "bf16 row stride": ("return oracle_bf16_to_f64(((const uint16_t *)W->w)[n * W->ldw + k]);",
                        "return oracle_bf16_to_f64(((const uint16_t *)W->w)[n * W->K + k]);"),
    "last k dropped": ("for (int64_t k = 0; k < W->K; k++) {", "for (int64_t k = 0; k < W->K - 1; k++) {"),
    "abs sum sign": ("acc_abs += fabs(p);", "acc_abs += p;"),
    "q8 rounding half to even": ("q[i] = (int8_t)roundf(v);", "q[i] = (int8_t)rintf(v);"),
    "q8 scale over 128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "q8 signed maximum": ("float a = fabsf(x[i]);", "float a = x[i];"),
    "mmq min term dropped": ("double term_m = a * ((double)mv * (double)sum);", "double term_m = 0.0;"),
    "mmq activation scale missing on the min term": ("double term_m = a * ((double)mv * (double)sum);",
                                                     "double term_m = (double)mv * (double)sum;"),
    "mmq chunk coefficients": ("oracle_q4k_coeffs(w, K, n, c, &dv, &mv); /* chunk c of row n */",
                               "oracle_q4k_coeffs(w, K, n, c / 2, &dv, &mv);"),
    "f32 rounding one significand bit short": (
        "double oracle_round_f32(double v) { return round_to_format(v, 24, -126, 0x1.FFFFFEp127); }",
        "double oracle_round_f32(double v) { return round_to_format(v, 23, -126, 0x1.FFFFFEp127); }"),
    "f32 rounding subnormal edge": (
        "double oracle_round_f32(double v) { return round_to_format(v, 24, -126, 0x1.FFFFFEp127); }",
        "double oracle_round_f32(double v) { return round_to_format(v, 24, -125, 0x1.FFFFFEp127); }"),
    "f32 rounding without overflow": (
        "double oracle_round_f32(double v) { return round_to_format(v, 24, -126, 0x1.FFFFFEp127); }",
        "double oracle_round_f32(double v) { return round_to_format(v, 24, -126, 0x1.FFFFFEp128); }"),
    "mmq activation index": ("dot += (int64_t)qw[k] * (int64_t)qa[t * K + k];",
                             "dot += (int64_t)qw[k] * (int64_t)qa[k];"),
}


def _run_pins(libpath):
    env = dict(os.environ, QGEMV_ORACLE_LIB=libpath)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared",
                           str(c), "-o", str(so), "-lm"])
    return str(so)


def test_unmodified_oracle_passes(tmp_path):
    with open(SRC) as f:
        src = f.read()
    assert _run_pins(_build(src, tmp_path, "orig")) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new, 1)
    if name == "plane row-major instead of chunk-major":
        mutated = mutated.replace("plane[(c * N + n) * 2 + 1] = mv;",
                                  "plane[(n * nchunk + c) * 2 + 1] = mv;", 1)
    assert _run_pins(_build(mutated, tmp_path, "mut")) != 0, f"pins missed mutant: {name}"
