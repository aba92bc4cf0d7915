"""Mutation test of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's C source
(a dropped term, a wrong sign, a wrong index or stride, a transposed operand,
a bad decoder constant, a missing guard), builds it with gcc in a temporary
directory, and runs the oracle pin suite against that build in a child
process.  The suite must fail for every mutant; the real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "softmax_oracle.c")

MUTANTS = {
    "no_max_subtraction": ("y[j] = exp(y[j] - m);", "y[j] = exp(y[j]);"),
    "wrong_sign": ("y[j] = exp(y[j] - m);", "y[j] = exp(m - y[j]);"),
    "dropped_first_term": ("s += y[j];", "if (j > 0) s += y[j];"),
    "stride_ignored": ("i * row_stride + j", "i * cols + j"),
    "transposed": ("i * row_stride + j", "j * row_stride + i"),
    "no_all_neg_inf_guard": ("if (m == -INFINITY) {", "if (0) {"),
    "max_off_by_one": ("for (int64_t j = 0; j < cols; ++j)\n            if (y[j] > m)",
                       "for (int64_t j = 1; j < cols; ++j)\n            if (y[j] > m)"),
    "f16_bias": ("expo - 25", "expo - 24"),
    "f16_subnormal": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "bf16_hidden_bit": ("(double)(128 + frac)", "(double)(frac)"),
    "multiply_by_sum": ("y[j] = y[j] / s;", "y[j] = y[j] * s;"),
    "causal_kept_off_by_one": ("kept = i + diag + 1;", "kept = i + diag;"),
    "causal_scale_dropped": ("y[j] = scale * load_element(in, dtype, i * row_stride + j);",
                             "y[j] = load_element(in, dtype, i * row_stride + j);"),
    "causal_reads_masked": ("for (int64_t j = 0; j < kept; ++j)\n            y[j] = scale",
                            "for (int64_t j = 0; j < cols; ++j)\n            y[j] = scale"),
    "causal_diag_sign": ("} else if (diag < -i) {", "} else if (diag < i) {"),
    "attn_scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "attn_causal_offset": ("kept = i + (nk - nq) + 1;", "kept = i + 1;"),
    "attn_k_from_q_base": ("* load_element(k, dtype, kb + j * d + c);", "* load_element(k, dtype, qb + j * d + c);"),
    "attn_v_transposed": ("o[c] += p * load_element(v, dtype, kb + j * d + c);",
                          "o[c] += p * load_element(v, dtype, kb + c * nk + j);"),
    "attn_unnormalised": ("const double p = s[j] / sum;", "const double p = s[j];"),
    "attn_no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "attn_first_query_only": ("load_element(q, dtype, qb + i * d + c)", "load_element(q, dtype, qb + c)"),
    "attn_causal_one_future_key": ("kept = i + (nk - nq) + 1;", "kept = i + (nk - nq) + 2;"),
    "attn_k_row_stride": ("* load_element(k, dtype, kb + j * d + c);", "* load_element(k, dtype, kb + j + c);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", "-o", str(lib), str(mutant_c), "-lm"],
                   check=True)
    env = dict(os.environ, ROW_SOFTMAX_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py"),
                        os.path.join(ROOT, "tests", "test_oracle_causal.py"),
                        os.path.join(ROOT, "tests", "test_oracle_attention.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
