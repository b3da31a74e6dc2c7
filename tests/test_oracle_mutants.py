"""Plant plausible mistakes in copies of the oracle's C source; the pins must catch
every one. The unmodified source, built the same way, must pass them all.

Each mutant is compiled to a temporary library and checked by tests/pin_suite.py in a
subprocess, so a mutant that crashes (e.g. by reading outside X) also counts as caught.
"""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

# (name, [(exact text in maxsim_oracle.c, replacement), ...])
MUTANTS = [
    ("max_becomes_min", [("double m = -INFINITY;", "double m = INFINITY;"),
                         ("if (dot > m)", "if (dot < m)")]),
    ("running_max_starts_at_zero", [("double m = -INFINITY;", "double m = 0.0;")]),
    ("stride_ignored", [("(off + t) * stride", "(off + t) * d")]),
    ("offset_ignored", [("(off + t) * stride", "(t) * stride")]),
    ("last_doc_row_dropped", [("t < len; ++t", "t + 1 < len; ++t")]),
    ("first_doc_row_dropped", [("int64_t t = 0; t < len", "int64_t t = 1; t < len")]),
    ("first_query_row_dropped", [("int32_t q = 0; q < Lq; ++q)", "int32_t q = 1; q < Lq; ++q)")]),
    ("doc_columns_reversed", [("tab[row[k]]", "tab[row[d - 1 - k]]")]),
    ("query_transposed", [("Qd[(int64_t)q * d + k]", "Qd[(int64_t)k * Lq + q]")]),
    ("sum_becomes_max", [("s += m;", "s = m > s ? m : s;")]),
    ("dot_in_fp32", [("double dot = 0.0;", "float dot = 0.0f;")]),
    ("offset_32bit", [("const uint16_t *row = X + (off + t) * stride;",
                       "const uint16_t *row = X + (int32_t)((off + t) * stride);")]),
    ("f16_bias_off_by_one", [("expo - 25)", "expo - 24)")]),
    ("f16_subnormals_flushed", [("v = ldexp((double)frac, -24);", "v = 0.0;")]),
    ("f16_sign_dropped", [("int sign = (h >> 15) & 1;", "int sign = 0;")]),
    ("f16_implicit_bit_dropped", [("(double)(1024 + frac)", "(double)(frac)")]),
    ("bf16_scale_off_by_one", [("expo - 134)", "expo - 133)")]),
    ("bf16_sign_dropped", [("int sign = (b >> 15) & 1;", "int sign = 0;")]),
    ("bf16_read_as_f16", [(": oracle_decode_bf16((uint16_t)u);", ": oracle_decode_f16((uint16_t)u);")]),
    # FP8 E4M3 doc storage
    ("e4m3_bias_of_fnuz", [("v = ldexp((double)(8 + frac), expo - 10);", "v = ldexp((double)(8 + frac), expo - 11);")]),
    ("e4m3_subnormals_flushed", [("v = ldexp((double)frac, -9);", "v = 0.0;")]),
    ("e4m3_no_nan", [("if (expo == 15 && frac == 7)\n        return NAN;", "")]),
    ("e4m3_sign_dropped", [("int sign = (b >> 7) & 1;", "int sign = 0;")]),
    ("fp8_scale_ignored", [("xtab[u] = doc_scale * oracle_decode_e4m3((uint8_t)u);",
                            "xtab[u] = oracle_decode_e4m3((uint8_t)u);")]),
    ("fp8_stride_ignored", [("const uint8_t *row = X + (off + t) * stride;",
                             "const uint8_t *row = X + (off + t) * d;")]),
    ("fp8_query_read_as_other_format", [("oracle_decode_table(qfmt, tab);", "oracle_decode_table(1 - qfmt, tab);")]),
]


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, os.path.join(HERE, "pin_suite.py"), lib],
                          capture_output=True, text=True, timeout=300)


def _build(src_text: str, tmp_path, name: str) -> str:
    src = tmp_path / f"{name}.c"
    src.write_text(src_text)
    lib = str(tmp_path / f"lib{name}.so")
    oracle.compile_source(str(src), lib)
    return lib


def test_unmodified_oracle_passes_pin_suite(tmp_path):
    text = open(oracle.SOURCE).read()
    res = _run_pins(_build(text, tmp_path, "control"))
    assert res.returncode == 0, res.stdout + res.stderr


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, edits, tmp_path):
    text = open(oracle.SOURCE).read()
    for old, new in edits:
        # A site shared by the fp16/bf16 and the FP8 loops is mutated in both.
        assert text.count(old) >= 1, f"mutation site {old!r} not in the oracle source"
        text = text.replace(old, new)
    res = _run_pins(_build(text, tmp_path, name))
    assert res.returncode != 0, f"mutant {name} survived the pins:\n{res.stdout}{res.stderr}"
