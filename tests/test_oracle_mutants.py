"""The oracle's pins must catch plausible mistakes.

Each case compiles a copy of the oracle's C source with one deliberate
mistake (on the CPU, into a temporary directory) and runs the pin suite
(tests/test_oracle.py) against it in a subprocess; the suite must fail.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "q4_oracle.c")

MUTANTS = {
    "nibble_order_swapped": ("(byte & 0x0F) : (byte >> 4)", "(byte >> 4) : (byte & 0x0F)"),
    "offset_7_not_8": ("code_at(wq_row, k) - 8) * fp16_value(ws_row", "code_at(wq_row, k) - 7) * fp16_value(ws_row"),
    "scale_block_64": ("ws_row[k / Q4O_BLOCK]", "ws_row[k / 64]"),
    "fp16_exponent_bias": ("e - 25);", "e - 24);"),
    "fp16_subnormal_quantum": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_exponent_bias": ("e - 134);", "e - 133);"),
    "output_transposed": ("K, bf16_weights,\n                    &y[m * N + n], &t[m * N + n]",
                          "K, bf16_weights,\n                    &y[n * M + m], &t[n * M + m]"),
    "sum_sign": ("acc += p;\n        mag += fabs(p);\n    }", "acc -= p;\n        mag += fabs(p);\n    }"),
    "abs_dropped": ("mag += fabs(p);\n    }", "mag += p;\n    }"),
    "bf16_round_truncates": ("r = ldexp(rint(ldexp(a, 8 - e)), e - 8);",
                             "r = ldexp(floor(ldexp(a, 8 - e)), e - 8);"),
    "moe_gate_dropped": ("acc += g * d;", "acc += d;"),
    "moe_abs_gate_dropped": ("mag += fabs(g) * dm;", "mag += dm;"),
}


# Mutants of the 4-bit float block product, run against tests/test_oracle_mx.py.
MX_MUTANTS = {
    "mx_exponent_bias_0": ("ldexp(2.0 + m, e - 2)", "ldexp(2.0 + m, e - 1)"),
    "mx_sign_bit_0": ("int sign = (c >> 3) & 1;\n    int e = (c >> 1) & 3;\n    int m = c & 1;",
                      "int sign = c & 1;\n    int e = (c >> 1) & 3;\n    int m = (c >> 3) & 1;"),
    "mx_subnormal_weight": ("ldexp((double)m, -1)", "ldexp((double)m, 0)"),
    "mx_scale_bias_128": ("ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 128)"),
    "mx_scale_block_16": ("we_row[k / Q4O_BLOCK]", "we_row[k / 16]"),
}


# Mutants of the routed FFN, run against tests/test_oracle_ffn.py.
FFN_MUTANTS = {
    "ffn_gate_up_swapped": ("int64_t rg = e * 2 * F + 2 * f, ru = rg + 1;",
                            "int64_t ru = e * 2 * F + 2 * f, rg = ru + 1;"),
    "ffn_silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "ffn_silu_dropped": ("double sg = silu(gv);", "double sg = gv;"),
    "ffn_route_weight_dropped": ("y[tok * H + h] += g * o;", "y[tok * H + h] += o;"),
    "ffn_down_rows_transposed": ("const uint8_t *wr = w2q + (e * H + h) * (F / 2);",
                                 "const uint8_t *wr = w2q + (h * E + e) * (F / 2);"),
    "ffn_bound_propagation_dropped": (
        "da[f] = fabs(a[f]) + 1.1 * fabs(uv) * tg + fabs(sg) * tu;", "da[f] = fabs(a[f]);"),
}


# Mutants of the RMSNorm prologue, run against tests/test_oracle_rmsnorm.py.
RMS_MUTANTS = {
    "rms_eps_dropped": ("double r = 1.0 / sqrt(ss / (double)K + eps);",
                        "double r = 1.0 / sqrt(ss / (double)K);"),
    "rms_sum_not_mean": ("double r = 1.0 / sqrt(ss / (double)K + eps);",
                         "double r = 1.0 / sqrt(ss + eps);"),
    "rms_sqrt_dropped": ("double r = 1.0 / sqrt(ss / (double)K + eps);",
                         "double r = 1.0 / (ss / (double)K + eps);"),
    "rms_gamma_dropped": ("xn[m * K + k] = bf16_value(x[m * K + k]) * r * bf16_value(gamma[k]);",
                          "xn[m * K + k] = bf16_value(x[m * K + k]) * r;"),
    "rms_gamma_index": ("xn[m * K + k] = bf16_value(x[m * K + k]) * r * bf16_value(gamma[k]);",
                        "xn[m * K + k] = bf16_value(x[m * K + k]) * r * bf16_value(gamma[K - 1 - k]);"),
    "rms_half_ulp_double": ("return ldexp(1.0, (e - 1) - 8);", "return ldexp(1.0, (e - 1) - 7);"),
    "rms_abs_dropped": ("        mag += fabs(p);\n        rnd +=", "        mag += p;\n        rnd +="),
}


# Mutants of the quantiser, run against tests/test_oracle_quantize.py.
QUANT_MUTANTS = {
    "q_max_by_value": ("if (fabs(v) > fabs(m))", "if (v > m)"),
    "q_divisor_sign": ("fp16_round_clamped(m / -8.0)", "fp16_round_clamped(m / 8.0)"),
    "q_offset_7": ("fminf(15.0f, q + 8.0f)", "fminf(15.0f, q + 7.0f)"),
    "q_round_down": ("rintf((float)bf16_value(blk[i]) / (float)s)",
                     "floorf((float)bf16_value(blk[i]) / (float)s)"),
    # m / -8 has at most 8 significant bits, so only fp16's subnormal range
    # rounds it
    "q_fp16_subnormal_truncates": ("r = ldexp(rint(ldexp(a, 24)), -24);",
                                   "r = ldexp(floor(ldexp(a, 24)), -24);"),
    "q_nibble_order": ("if (k % 2 == 0)\n                    *byte", "if (k % 2 == 1)\n                    *byte"),
    "q_clamp_14": ("fminf(15.0f, q + 8.0f)", "fminf(14.0f, q + 8.0f)"),
}


# Mutants of the super-block scale format, run against tests/test_oracle_sb.py.
SB_MUTANTS = {
    "sb_super_index_128": ("fp16_value(wd_row[k / 256])", "fp16_value(wd_row[k / 128])"),
    "sb_multiplier_dropped": ("fp16_value(wd_row[k / 256]) *\n           (double)wsc_row[k / Q4O_BLOCK];",
                              "fp16_value(wd_row[k / 256]);"),
    "sb_multiplier_index": ("(double)wsc_row[k / Q4O_BLOCK];", "(double)wsc_row[k / 64];"),
    "sb_offset_7": ("return (double)(code_at(wq_row, k) - 8) * fp16_value(wd_row",
                    "return (double)(code_at(wq_row, k) - 7) * fp16_value(wd_row"),
    "sb_abs_dropped": ("                sum += p;\n                mag += fabs(p);",
                       "                sum += p;\n                mag += p;"),
}


def _run_suite_on_mutant(old, new, suite, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.compile_to(str(mpath), lib)
    env = dict(os.environ, Q4_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", suite)],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(MX_MUTANTS))
def test_mx_pins_catch_mutant(name, tmp_path):
    r = _run_suite_on_mutant(*MX_MUTANTS[name], "test_oracle_mx.py", tmp_path)
    assert r.returncode != 0, f"mutant {name} passed every 4-bit float pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(FFN_MUTANTS))
def test_ffn_pins_catch_mutant(name, tmp_path):
    r = _run_suite_on_mutant(*FFN_MUTANTS[name], "test_oracle_ffn.py", tmp_path)
    assert r.returncode != 0, f"mutant {name} passed every FFN pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.compile_to(str(mpath), lib)
    env = dict(os.environ, Q4_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(RMS_MUTANTS))
def test_rms_pins_catch_mutant(name, tmp_path):
    r = _run_suite_on_mutant(*RMS_MUTANTS[name], "test_oracle_rmsnorm.py", tmp_path)
    assert r.returncode != 0, f"mutant {name} passed every RMSNorm pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quant_pins_catch_mutant(name, tmp_path):
    r = _run_suite_on_mutant(*QUANT_MUTANTS[name], "test_oracle_quantize.py", tmp_path)
    assert r.returncode != 0, f"mutant {name} passed every quantiser pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(SB_MUTANTS))
def test_sb_pins_catch_mutant(name, tmp_path):
    r = _run_suite_on_mutant(*SB_MUTANTS[name], "test_oracle_sb.py", tmp_path)
    assert r.returncode != 0, f"mutant {name} passed every super-block pin:\n{r.stdout[-2000:]}"
