"""The oracle's pins must reject a wrong oracle (CPU only).

Each case plants one plausible mistake in a copy of oracle/qsa_oracle.c --
a dropped term, a wrong sign, scale or index, a transposed operand, the
wrong tie rule, a missing sort, a wrong rounding -- builds it with gcc, and
runs the pin files (tests/test_oracle_pins.py, tests/test_oracle_quantize_pins.py)
in a child process whose oracle loads that build.  At least one pin must
fail; a planted mistake that every pin lets through would mean a gap in
them.  The oracle itself is never changed: the copies live in a temporary
directory.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qsa_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_oracle_quantize_pins.py")]

# name -> (text in qsa_oracle.c, its replacement); each text occurs once
MUTANTS = {
    # softmax temperature: 1/D instead of 1/sqrt(D)
    "score_scale": ("const double scale = 1.0 / sqrt((double)D); /* 0.0625 at D = 256 */",
                    "const double scale = 1.0 / (double)D; /* 0.0625 at D = 256 */"),
    # visible cells: the token itself left out
    "visible_cells": ("  int64_t n = (int64_t)pos0 + t + 1;\n  return n <= budget ? n : budget;",
                      "  int64_t n = (int64_t)pos0 + t;\n  return n <= budget ? n : budget;"),
    # ties to the higher index
    "tie_rule": ("return (a->c < b->c) ? -1 : (a->c > b->c);",
                 "return (a->c > b->c) ? -1 : (a->c < b->c);"),
    # selected ids left in score order
    "ids_unsorted": ("    qsort(row, (size_t)budget, sizeof(int32_t), by_int_asc);\n", "\n"),
    # a row at exactly the budget reads its ids instead of the identity
    "identity_edge": ("  if (n <= budget) return i;", "  if (n < budget) return i;"),
    # softmax denominator counts cells instead of summing weights
    "softmax_sum": ("        s[i] = exp(s[i] - m);\n        l += s[i];",
                    "        s[i] = exp(s[i] - m);\n        l += 1.0;"),
    # K scale block taken by the wrong index
    "k_scale_block": ("acc += qh[d] * ((double)kc[d] * sc[d / blk]);",
                      "acc += qh[d] * ((double)kc[d] * sc[d % nblk]);"),
    # keys in place of values in the weighted sum
    "v_is_k": ("        const int8_t *vc = vq_g + c * D;\n        const double *sc = vsc_g + c * nblk;\n"
               "        for (int d = 0; d < D; ++d) oh[d] +=",
               "        const int8_t *vc = kq_g + c * D;\n        const double *sc = vsc_g + c * nblk;\n"
               "        for (int d = 0; d < D; ++d) oh[d] +="),
    # V scale of the wrong sign
    "v_scale_sign": ("oh[d] += s[i] * ((double)vc[d] * sc[d / 64]);",
                     "oh[d] += s[i] * ((double)vc[d] * -sc[d / 64]);"),
    # chunk partial: m shifted away from the chunk's max
    "partial_max": ("        m[rec] = mk;", "        m[rec] = mk + 0.5;"),
    # merge: records summed without their e^(m_k - M) factor
    "merge_factor": ("for (int d = 0; d < D; ++d) oh[d] += e * (double)rec[d];",
                     "for (int d = 0; d < D; ++d) oh[d] += (double)rec[d];"),
    # merge: sign of the exponent flipped
    "merge_sign": ("double e = exp((double)rec[D] - M);", "double e = exp(M - (double)rec[D]);"),
    # selection score: the first term of the dot product dropped
    "score_term": ("for (int d = 0; d < D; ++d) acc += q[d] * p[d];",
                   "for (int d = 1; d < D; ++d) acc += q[d] * p[d];"),
    # quantiser: absmax over 128 instead of 127
    "quant_scale": ("f32_to_f16_bits_rne(amax / 127.0f)", "f32_to_f16_bits_rne(amax / 128.0f)"),
    # quantiser: ties away from zero instead of to even
    "quant_ties": ("c = rintf(f16_bits_to_f32(xb[d]) / s);",
                   "c = roundf(f16_bits_to_f32(xb[d]) / s);"),
    # quantiser: no clamp at -127
    "quant_clamp": ("          if (c < -127.0f) c = -127.0f;\n", "\n"),
    # fp16 rounding by truncation
    "f16_truncate": ("const float m = rintf(ldexpf(fr, 11));", "const float m = truncf(ldexpf(fr, 11));"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_a_planted_mistake(name, tmp_path):
    with open(SRC) as f:
        src = f.read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "the mutation site must occur once in qsa_oracle.c"
    c_path = tmp_path / "qsa_oracle_mutant.c"
    c_path.write_text(src.replace(old, new))
    so_path = tmp_path / "libqsa_oracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                    str(so_path), str(c_path), "-lm"], check=True)
    env = dict(os.environ, QSA_ORACLE_MUTANT_LIB=str(so_path), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-1500:]
    # pytest exit status 1: the run completed and a test failed (not a
    # collection or usage error, which would be 2-5)
    assert r.returncode == 1, "every pin passed with mistake %r planted:\n%s" % (name, tail)
    assert " failed" in r.stdout, tail
