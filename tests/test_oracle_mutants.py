"""Plant mistakes in copies of the oracle (on the CPU) and check the pins catch each.

Each mutant is a one-token edit of ``oracle/il_oracle.c`` of the kind a
careless implementation could contain: a swapped nibble order, a wrong
offset, a dropped term, a wrong index, a transposed output, a wrong bias.
The mutant is compiled to a scratch library and the pin suite
(``tests/oracle_pins.py``) runs against it in a child process; the test
passes when at least one pin fails (or the child crashes).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    "q4_nibble_order": ("(e % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
                        "(e % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    "q4_offset": ("(double)(code - 8)", "(double)(code - 7)"),
    "q4_scale_block": ("double scale = orc_f16_value(rd_u16(blk));",
                       "double scale = orc_f16_value(rd_u16(base + (size_t)r * (size_t)nb * "
                       "ORC_Q4_BLOCK_BYTES));"),
    "q8_code_offset": ("(int8_t)blk[4 + e]", "(int8_t)blk[3 + e]"),
    "q8_unsigned_code": ("(float)(int8_t)blk[4 + e]", "(float)blk[4 + e]"),
    "q8_scale_endian": ("uint32_t u = (uint32_t)p[0] |", "uint32_t u = (uint32_t)p[3] |"),
    "bf16_bias": ("ldexp((double)(128 + f), e - 127 - 7)", "ldexp((double)(128 + f), e - 126 - 7)"),
    "bf16_subnormal": ("ldexp((double)f, -126 - 7)", "ldexp((double)f, -126 - 8)"),
    "f16_subnormal": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "f16_bias": ("e - 15 - 10", "e - 14 - 10"),
    "dropped_first_term": ("for (int64_t k = 0; k < n_in; ++k) {\n                        double p",
                           "for (int64_t k = 1; k < n_in; ++k) {\n                        double p"),
    "dropped_last_term": ("for (int64_t k = 0; k < n_in; ++k) {\n                        double p",
                          "for (int64_t k = 0; k < n_in - 1; ++k) {\n                        double p"),
    "x_row_index": ("const float *xi = x + (size_t)i * (size_t)n_in;", "const float *xi = x;"),
    "bound_signed": ("mag += fabs(p);\n                    }\n                    y[",
                     "mag += p;\n                    }\n                    y["),
    "subset_row_offset": ("orc_dequant_row(weight, fmt, n_in, r0 + j, w)",
                          "orc_dequant_row(weight, fmt, n_in, j, w)"),
    "y_transposed": ("y[(size_t)i * (size_t)nr + (size_t)j] = (float)acc;",
                     "y[(size_t)j * (size_t)t + (size_t)i] = (float)acc;"),
    "product_sign": ("double p = (double)xi[k] * (double)w[k];",
                     "double p = -(double)xi[k] * (double)w[k];"),
    "points_x_row": ("const float *xi = x + (size_t)ii[p] * (size_t)n_in;", "const float *xi = x;"),
    "check_loose": ("ok = (err <= tol * bound[e]);", "ok = (err <= 2 * tol * bound[e]);"),
    "check_zero_bound": ("ok = (err == 0.0);", "ok = 1;"),
    "f16_round_down": ("double f = nearbyint((2.0 * m - 1.0) * 1024.0);",
                       "double f = floor((2.0 * m - 1.0) * 1024.0);"),
    "f16_subnormal_round_down": ("double q = nearbyint(a * ldexp(1.0, 24));",
                                 "double q = floor(a * ldexp(1.0, 24));"),
    "f16_overflow": ("if (be >= 31) return sign", "if (be >= 32) return sign"),
    "gelu_x_row": ("const float *xrow = x + (size_t)i * (size_t)n_in;", "const float *xrow = x;"),
    "lm_tie_index": ("(vb == vbest && idx[b] < idx[best])", "(vb == vbest && idx[b] > idx[best])"),
    "lm_select_smallest": ("if (vb > vbest ||", "if (vb < vbest ||"),
    "lm_last_max": ("if (best_tok < 0 || sc > best_s) {", "if (best_tok < 0 || sc >= best_s) {"),
    "lm_ordering_index": ("const uint32_t tok = ordering[c * per + j];", "const uint32_t tok = ordering[j * n_c + c];"),
    "lm_token_row_offset": ("embed + (size_t)tok * (size_t)h, x, h, bound", "embed + (size_t)tok, x, h, bound"),
    "lm_token_bound_signed": ("        m += fabs(p);", "        m += p;"),
    "lm_topk_unclamped": ("if (k > n_c) k = n_c;", "if (k > n_c) return -1;"),
    "lm_x_row": ("const float *xi = x + (size_t)i * (size_t)h;", "const float *xi = x;"),
    "gelu_half": ("return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));", "return v * (1.0 + erf(v / sqrt(2.0)));"),
    "gelu_erf_argument": ("erf(v / sqrt(2.0))", "erf(v)"),
    "gelu_mul_operand": ("double v = gl * u;", "double v = gl * g;"),
    "gelu_up_row": ("orc_dequant_row(up, fmt, n_in, r0 + j, wu)", "orc_dequant_row(gate, fmt, n_in, r0 + j, wu)"),
    "gelu_bound_up_term": ("+ fabs(gl) * tau * bu +", "+"),
    "gelu_bound_slope": ("const double tau = 4e-3, lip = 1.13;", "const double tau = 4e-3, lip = 1.0;"),
    "quant_q8_divisor": ("float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    "quant_q8_truncate": ("q = rintf(src[e] / s);\n                        if (q > 127.0f)",
                          "q = truncf(src[e] / s);\n                        if (q > 127.0f)"),
    "quant_q4_divisor": ("orc_f16_bits(amax / 7.0f)", "orc_f16_bits(amax / 8.0f)"),
    "quant_q4_nibbles": ("(e % 2 == 0) ? code : code << 4", "(e % 2 == 0) ? code << 4 : code"),
    "quant_q4_unrounded_scale": ("float s = (float)orc_f16_value(sb);", "float s = amax / 7.0f;"),
}

_CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {here!r}]
import oracle, oracle_pins
failed = oracle_pins.run_all(oracle.Oracle({so!r}), quick=True)
print("\n".join(failed))
sys.exit(1 if failed else 0)
"""


def _run_child(so):
    child = _CHILD.format(root=ROOT, here=HERE, so=so)
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout + r.stderr[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Compile every mutant and run the pin suite on each, several at a time."""
    src = open(oracle.SRC).read()
    d = tmp_path_factory.mktemp("mutants")
    jobs = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not unique/found"
        c = d / f"{name}.c"
        c.write_text(src.replace(old, new))
        jobs[name] = oracle.compile_oracle(str(c), str(d / f"lib{name}.so"))
    jobs["(unmutated)"] = oracle.compile_oracle(oracle.SRC, str(d / "libclean.so"))
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {name: ex.submit(_run_child, so) for name, so in jobs.items()}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, mutant_results):
    rc, out = mutant_results[name]
    assert rc != 0, f"mutant {name} passed every pin:\n{out}"


def test_unmutated_passes_quick_suite(mutant_results):
    rc, out = mutant_results["(unmutated)"]
    assert rc == 0, out
