"""Each plausible mistake planted in a copy of the oracle must be caught by at least one pin.

The copies are built with gcc into a temporary directory and exercised in a child process (a
planted mistake may read out of bounds; a crash then only ends the child).  A mutant counts as
caught when the child names at least one failed pin, or when it is ended by a signal; any other
failure of the child is a failure of the harness.  CPU only.
"""

import json
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fa_oracle.c")

# (name, text in fa_oracle.c, replacement)
MUTANTS = [
    ("gqa_head_modulo", "const int64_t kvh = h / group;", "const int64_t kvh = h % p->kv_heads;"),
    ("dropped_scale", "double s = p->scale * dot;", "double s = dot;"),
    ("causal_off_by_one", "if (p->causal && j > cmax) attended = 0;",
     "if (p->causal && j >= cmax) attended = 0;"),
    ("causal_top_left", ": L - p->sq + i;", ": i;"),
    ("window_off_by_one", "lo = cmax + 1 - p->local_window;", "lo = cmax - p->local_window;"),
    ("window_when_disabled", "if (p->local_window > 0) {", "if (p->local_window >= 0) {"),
    ("softcap_after_mask",
     "        if (p->softcap > 0.0) s = p->softcap * tanh(s / p->softcap);\n"
     "        if (plane >= 0) s += (double)p->mask[(plane * p->sq + i) * p->sk + j];",
     "        if (plane >= 0) s += (double)p->mask[(plane * p->sq + i) * p->sk + j];\n"
     "        if (p->softcap > 0.0) s = p->softcap * tanh(s / p->softcap);"),
    ("mask_transposed", "(plane * p->sq + i) * p->sk + j", "(plane * p->sk + j) * p->sq + i"),
    ("mask_batch_plane_ignored", "if (p->mask_planes == p->batch) return b;",
     "if (p->mask_planes == p->batch) return 0;"),
    ("mask_head_plane_swapped", "return b * p->heads + h;", "return h * p->batch + b;"),
    ("score_sign", "x[j] = exp(x[j] - m);", "x[j] = exp(m - x[j]);"),
    ("minus_inf_kept", "keep[j] = (s != -INFINITY);", "keep[j] = 1;"),
    ("token_major_as_head_major",
     "dst = w->out + ((b * p->sq + i) * p->heads + h) * p->dim;",
     "dst = w->out + ((b * p->heads + h) * p->sq + i) * p->dim;"),
    ("kv_plane_stride_sk",
     "const float* kbase = p->k + (b * p->kv_heads + kvh) * p->kv_capacity * D;",
     "const float* kbase = p->k + (b * p->kv_heads + kvh) * p->sk * D;"),
    ("total_lengths_ignored", "if (p->total_lengths != NULL && (int64_t)",
     "if (0 && (int64_t)"),
    ("past_lengths_ignored", "const int64_t cmax = p->past_lengths != NULL ?",
     "const int64_t cmax = 0 ?"),
    ("no_normalisation", "const double w = x[j] / denom;", "const double w = x[j];"),
    ("query_uses_kv_head", "const float* qrow = p->q + ((b * p->heads + h) * p->sq + i) * D;",
     "const float* qrow = p->q + ((b * p->heads + kvh) * p->sq + i) * D;"),
    ("values_from_keys", "o[d] += w * (double)vbase[j * D + d];",
     "o[d] += w * (double)kbase[j * D + d];"),
    # the causal base from the uncapped total length (the other reading of total > sk)
    ("causal_base_uncapped_total", ": L - p->sq + i;",
     ": (p->total_lengths != NULL ? (int64_t)p->total_lengths[b] : p->sk) - p->sq + i;"),
    ("total_not_capped_at_sk", "(int64_t)p->total_lengths[b] < L) L = p->total_lengths[b];",
     "(int64_t)p->total_lengths[b] != L) L = p->total_lengths[b];"),
]

_DRIVER = r"""
import json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
from oracle_pins import ALL_PINS
orc = oracle.Oracle({lib!r})
failed = []
for pin in ALL_PINS:
    try:
        pin(orc)
    except Exception as exc:  # an assertion, or a rejected/NaN-producing problem
        failed.append(pin.__name__)
print("FAILED_PINS=" + json.dumps(failed))
"""


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(source, name, old, new, tmp_path):
    assert source.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    import oracle

    mutated = source.replace(old, new)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(src), lib)
    driver = _DRIVER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    proc = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True,
                          timeout=300)
    if proc.returncode < 0:
        return  # the planted mistake crashed the oracle (the child ended by a signal): caught
    # anything else must be a clean run of the driver that names the failed pins; an import
    # error or another failure of the harness itself is not a catch
    assert proc.returncode == 0, f"the pin driver failed for {name}:\n{proc.stdout}{proc.stderr}"
    line = [ln for ln in proc.stdout.splitlines() if ln.startswith("FAILED_PINS=")]
    assert line, proc.stdout + proc.stderr
    failed = json.loads(line[-1].split("=", 1)[1])
    assert failed, f"no pin caught the planted mistake {name}"
