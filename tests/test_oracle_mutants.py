"""Planted mistakes in copies of the oracle (CPU only) must each be caught by a pin.

Each mutant is the oracle source with one plausible slip applied as a text
edit, compiled into a temporary directory.  The real oracle is not modified.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "no_logit_scale": ("double scale = 1.0 / sqrt((double)dh);", "double scale = 1.0;"),
    "k_reads_q": ("+ c->d + (int64_t)h * dh; /* K block */", "+ (int64_t)h * dh; /* K block */"),
    "v_ignores_head": ("2 * (int64_t)c->d + (int64_t)h * dh + e]", "2 * (int64_t)c->d + e]"),
    "no_normalise": ("oi[e] = acc / den;", "oi[e] = acc;"),
    "no_residual": ("c->x[t * (int64_t)c->d + n] + acc;", "acc;"),
    "wo_transposed": ("acc += orow[j] * wr[j];", "acc += orow[j] * c->Wo[(int64_t)j * c->d + n];"),
    "last_key_dropped": ("for (int64_t l = 0; l < L; ++l) {\n      const double* kl",
                         "for (int64_t l = 0; l < L - (L > 1); ++l) {\n      const double* kl"),
    "tail_window_backed_off": ("len[b] = (r + B <= end) ? B : end - r;",
                               "len[b] = (r + B <= end || r - a < B) ? (r + B <= end ? B : end - r) : B;\n"
                               "      if (r + B > end && r - a >= B) start[b] = end - B;"),
    "blocks_shifted": ("start[b] = r;", "start[b] = r > a ? r - 1 : r;"),
    "softmax_max_only_first": ("if (z[l] > m) m = z[l];", "if (z[l] > m) m = m;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant_src), str(tmp_path / "libmutant.so"))
    run = subprocess.run([sys.executable, "-m", "tests.run_pins", lib], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    if run.returncode != 0:
        failures = ["<crashed>"]
    else:
        failures = json.loads(run.stdout.strip().splitlines()[-1])
    if name == "softmax_max_only_first":
        # subtracting any finite constant before exp is exact in real arithmetic;
        # this edit is harmless and must not trip the value pins
        assert not failures, failures
        return
    assert failures, f"no pin caught mutant {name}"
