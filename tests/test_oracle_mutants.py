"""The oracle's pins must catch plausible slips.

Each case copies ttt_oracle.c, plants one slip (a wrong index, sign, dropped
term, transposed operand, inclusive instead of exclusive prefix, ...), builds
the copy on the CPU and runs the pin suite against it: the suite must fail.
Nothing here touches the GPU or the HIP library.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ttt_oracle.c")

MUTANTS = {
    "conv_no_lookahead": ("int64_t src = t + 1 - k;", "int64_t src = t - k;"),
    "silu_sign": ("x / (1.0 + exp(-x))", "x / (1.0 + exp(x))"),
    "dropped_up_projection": ("Z[t * f + n] = silu(a) * b;", "Z[t * f + n] = silu(a);"),
    "update_sign": ("W[m * f + n] += eta * s;", "W[m * f + n] -= eta * s;"),
    "no_update": ("W[m * f + n] += eta * s;", "W[m * f + n] += 0.0 * s;"),
    "target_transposed": ("s += U[t * d + c] * (double)Wt[c * d + j];",
                          "s += U[t * d + c] * (double)Wt[j * d + c];"),
    "dropped_first_tap": ("for (int32_t k = 0; k < K; ++k) {\n        int64_t src",
                          "for (int32_t k = 1; k < K; ++k) {\n        int64_t src"),
    "inclusive_prefix": ("P[(i - 1) * d * f + e] + dW[(i - 1) * d * f + e];",
                         "P[(i - 1) * d * f + e] + dW[i * d * f + e];"),
    "dual_token_causal": ("const int64_t ct = C * (t / C);", "const int64_t ct = t;"),
    "output_with_w0_only": ("s += Zc[r * f + n] * W[m * f + n];",
                            "s += Zc[r * f + n] * (double)0.0 + Zc[r * f + n] * W[m * f + n] * (r0 == 0);"),
}


def _build(src_text, path):
    c = path + ".c"
    with open(c, "w") as fh:
        fh.write(src_text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", path, c,
                    "-lm"], check=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_slip(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor not found for {name}"
    mutated = text.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as td:
        lib = os.path.join(td, "libmutant.so")
        _build(mutated, lib)
        env = dict(os.environ, TTT_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
