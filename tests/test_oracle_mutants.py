"""Planted mistakes in the oracle (on the CPU): every plausible slip in its
decoding, addressing, contraction or epilogue must make at least one pin
fail.  Each mutant is the oracle's C text with one edit, built into a
temporary library; the real oracle is never modified."""
import os
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = open(os.path.join(os.path.dirname(oracle.__file__),
                        "gemm_epi_oracle.c")).read()

# (name, original text, planted text)
MUTANTS = [
    ("f16_bias", "e - 25); /* (1+f/2^10)", "e - 24); /* (1+f/2^10)"),
    ("f16_subnormal", "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    ("f16_no_inf", "v = (f == 0) ? INFINITY : NAN;\n  else\n    v = ldexp((double)(1024",
     "v = ldexp((double)(1024 + f), e - 25);\n  else\n    v = ldexp((double)(1024"),
    ("bf16_bias", "e - 134)", "e - 133)"),
    ("bf16_subnormal", "ldexp((double)f, -133)", "ldexp((double)f, -126)"),
    ("e4m3_bias", "e - 10)", "e - 11)"),
    ("e4m3_nan_missing", "if (e == 15 && f == 7)", "if (0)"),
    ("e4m3_subnormal", "ldexp((double)f, -9)", "ldexp((double)f, -10)"),
    ("sign_dropped", "return s ? -v : v;\n}\n\nstatic double dec_bf16",
     "return v;\n}\n\nstatic double dec_bf16"),
    ("a_index_transposed", "m * d->K + k);", "k * d->M + m);"),
    ("a_mmajor_index", "k * d->M + m :", "m * d->K + k :"),
    ("a_batch_stride", "l * d->M * d->K +", "l * d->M * d->N +"),
    ("b_index_nmajor", "k * d->N + n :", "n * d->K + k :"),
    ("b_batch_stride", "l * d->N * d->K +", "l * d->M * d->K +"),
    ("cd_mmajor_index", "n * d->M + m :", "n * d->N + m :"),
    ("k_off_by_one", "k < d->K; ++k", "k < d->K - 1; ++k"),
    ("k_starts_at_one", "int64_t k = 0; k < d->K", "int64_t k = 1; k < d->K"),
    ("side_sum_signed", "s += fabs(a) * fabs(b);", "s += a * b;"),
    ("x_term_dropped", "out += p->xf * load(p->X, d->x_type, o);", "(void)o;"),
    ("beta_sign", "out += p->beta * load(", "out -= p->beta * load("),
    ("alpha_on_c", "double out = p->alpha * acc;", "double out = acc;"),
    ("beta_skip_ignored", "p->beta != 0.0)", "1)"),
    ("x_uses_c_type", "load(p->X, d->x_type, o)", "load(p->X, d->c_type, o)"),
    ("y_is_d", "if (yref) *yref = acc;", "if (yref) *yref = out;"),
    ("i8_unsigned", "(double)((const int8_t*)p)[i]", "(double)((const uint8_t*)p)[i]"),
    ("u8_signed", "case ORC_U8: return (double)((const uint8_t*)p)[i];",
     "case ORC_U8: return (double)((const int8_t*)p)[i];"),
    ("bf16_as_f16", "case ORC_BF16: return dec_bf16(", "case ORC_BF16: return dec_f16("),
    ("points_swap_mn", "element(j->p, q[0], q[1], q[2]", "element(j->p, q[0], q[2], q[1]"),
    ("e5m2_bias", "ldexp((double)(4 + f), e - 17)", "ldexp((double)(4 + f), e - 16)"),
    ("e5m2_subnormal", "ldexp((double)f, -16)", "ldexp((double)f, -17)"),
    ("e5m2_as_e4m3_fields", "e = (b >> 2) & 31, f = b & 3", "e = (b >> 3) & 15, f = b & 7"),
    ("b_uses_a_type", "load(p->B, d->b_type ? d->b_type : d->ab_type,", "load(p->B, d->ab_type,"),
    ("relu_ignored", "if (p->relu && !(out > 0.0)) out = 0.0;", "(void)0;"),
    ("relu_always", "if (p->relu && !(out > 0.0))", "if (!(out > 0.0))"),
    ("relu_keeps_negatives", "if (p->relu && !(out > 0.0)) out = 0.0;",
     "if (p->relu && (out > 0.0)) out = 0.0;"),
    ("relu_after_x",
     "  if (p->relu && !(out > 0.0)) out = 0.0;\n  if (p->X && d->x_type != ORC_NONE && p->xf != 0.0)\n"
     "    out += p->xf * load(p->X, d->x_type, o);",
     "  if (p->X && d->x_type != ORC_NONE && p->xf != 0.0)\n"
     "    out += p->xf * load(p->X, d->x_type, o);\n  if (p->relu && !(out > 0.0)) out = 0.0;"),
    ("relu_before_c", "  if (p->C && d->c_type != ORC_NONE && p->beta != 0.0)\n    out += p->beta * load(p->C, d->c_type, o);\n"
     "  if (p->relu && !(out > 0.0)) out = 0.0;",
     "  if (p->relu && !(out > 0.0)) out = 0.0;\n"
     "  if (p->C && d->c_type != ORC_NONE && p->beta != 0.0)\n    out += p->beta * load(p->C, d->c_type, o);"),
]


_RUNNER = r"""
import sys
sys.path[:0] = [%(root)r, %(tests)r]
import oracle
from oracle_pins import ALL_PINS
orc = oracle.Oracle(%(lib)r)
for pin in ALL_PINS:
    try:
        pin(orc)
    except Exception as e:
        print("CAUGHT", pin.__name__, type(e).__name__, flush=True)
"""


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, orig, planted):
    assert SRC.count(orig) == 1, "mutation anchor not unique: %s" % name
    path = oracle.compile_to(str(tmp_path / ("mut_%s.so" % name)),
                             SRC.replace(orig, planted))
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER % {"root": os.path.dirname(tests_dir), "tests": tests_dir,
                      "lib": path}
    # a child process: a mutant that writes out of bounds may crash, which
    # also counts as caught, but must not take the test runner down
    r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                       text=True, timeout=300)
    caught = [ln for ln in r.stdout.splitlines() if ln.startswith("CAUGHT")]
    assert caught or r.returncode != 0, \
        "planted mistake %s passed every pin" % name
