"""Each plausible mistake planted in a copy of the index-selection oracle must make at least one
of its pins (tests/test_dsa_oracle_pins.py) fail.  Copies are built with gcc in a temporary
directory and checked in a child pytest process.  A mutant counts as caught when that run ends
with failed pins, or when the child is ended by a signal; a collection or usage error is a
failure of the harness.  CPU only."""

import os
import re
import subprocess
import sys
import tempfile

import pytest

from oracle import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dsa_oracle.c")

MUTANTS = [
    ("fused_multiply_add",
     "const float prod = qrow[h * D + d] * krow[d];\n                        dot = dot + prod;",
     "dot = fmaf(qrow[h * D + d], krow[d], dot);"),
    ("head_dim_descending", "for (int64_t d = 0; d < D; ++d) {", "for (int64_t d = D - 1; d >= 0; --d) {"),
    ("heads_descending", "for (int64_t h = 0; h < H; ++h) {", "for (int64_t h = H - 1; h >= 0; --h) {"),
    ("relu_after_weighting", "const float term = relu(scaled) * wgt;", "const float term = relu(scaled * wgt);"),
    ("weights_scale_dropped", "const float wgt = wrow[h] * weights_scale;", "const float wgt = wrow[h];"),
    ("scale_dropped", "const float scaled = scale * dot;", "const float scaled = dot;"),
    ("allow_rule_inclusive", "if (!(bt > -1e30f)) {", "if (!(bt >= -1e30f)) {"),
    ("nan_not_canonical", "if (isnan(sc)) sc = canonical_nan();", ""),
    ("bias_not_added", "float sc = total + bt;", "float sc = total;"),
    ("key_of_batch_zero", "const float* krow = key + (b * T + t) * D;", "const float* krow = key + t * D;"),
    ("tie_to_higher_position", "return (x->pos > y->pos) - (x->pos < y->pos);",
     "return (x->pos < y->pos) - (x->pos > y->pos);"),
    ("picks_not_sorted", "qsort(pick, (size_t)keep, sizeof(int64_t), by_pos);", ""),
    ("sign_magnitude_order", "return (u & 0x80000000u) ? ~u : (u | 0x80000000u);", "return u ^ 0x80000000u;"),
    ("padding_zero", "out[r * top_k + i] = i < keep ? pick[i] : -1;", "out[r * top_k + i] = i < keep ? pick[i] : 0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    text = open(SRC).read()
    assert text.count(old) == 1, name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    dsa.build(str(src), lib)
    env = dict(os.environ, DSA_ORACLE_LIB=lib)
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_dsa_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    if proc.returncode < 0:
        return  # the planted mistake crashed the oracle (the child ended by a signal): caught
    # pytest exits with 1 when tests ran and some failed; 2-5 mean an interrupted run, an
    # internal or usage error, or no tests collected: failures of the harness, not catches
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout[-2000:]}"
    assert proc.returncode == 1 and re.search(r"\b\d+ failed\b", proc.stdout), (
        f"the pin run for mutant {name} did not end in failed pins (exit {proc.returncode}):\n"
        f"{proc.stdout[-2000:]}{proc.stderr[-2000:]}")
