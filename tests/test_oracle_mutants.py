"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle.c (on the CPU, in a
temporary directory), builds it, and runs tests/test_oracle_pins.py against
the mutant.  The pin suite must fail for every mutant.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "eps_outside_root": ("1.0 / sqrt(ss / (double)H + eps)", "1.0 / sqrt(ss / (double)H) + eps"),
    "divisor_H_minus_1": ("sqrt(ss / (double)H + eps)", "sqrt(ss / (double)(H > 1 ? H - 1 : 1) + eps)"),
    "gamma_reversed": ("y[j] = x[j] * r * gamma[j]", "y[j] = x[j] * r * gamma[H - 1 - j]"),
    "no_max_subtraction": ("for (int64_t j = 0; j < N; ++j) y[j] = exp(x[j] - m) / d;",
                           "for (int64_t j = 0; j < N; ++j) y[j] = exp(x[j]) / d;"),
    "dropped_term": ("for (int64_t j = 0; j < N; ++j) d += exp(x[j] - m);\n    for (int64_t j = 0; j < N; ++j) y[j]",
                     "for (int64_t j = 1; j < N; ++j) d += exp(x[j] - m);\n    for (int64_t j = 0; j < N; ++j) y[j]"),
    "wrong_sign": ("for (int64_t j = 0; j < N; ++j) y[j] = exp(x[j] - m) / d;",
                   "for (int64_t j = 0; j < N; ++j) y[j] = exp(m - x[j]) / d;"),
    "residual_unrounded": ("hr[j] = round_io(xr[j] + rr[j], io_dtype);", "hr[j] = xr[j] + rr[j];"),
    "bf16_double_rounding": ("if (isnan(v) || isinf(v) || v == 0.0) return v;",
                             "v = (double)(float)v;\n    if (isnan(v) || isinf(v) || v == 0.0) return v;"),
    "bf16_ties_away": ("double q = rint(v / spacing);", "double q = round(v / spacing);"),
    "bf16_one_bit_short": ("double spacing = ldexp(1.0, e - 7);", "double spacing = ldexp(1.0, e - 6);"),
    "ln_var_over_H_minus_1": ("double var = ss / (double)H;", "double var = ss / (double)(H > 1 ? H - 1 : 1);"),
    "ln_no_centering": ("y[j] = (x[j] - mu) * r * gamma[j]", "y[j] = x[j] * r * gamma[j]"),
    "ln_beta_dropped": ("+ (beta ? beta[j] : 0.0);", "+ 0.0;"),
    "ln_eps_outside": ("double r = 1.0 / sqrt(var + eps);", "double r = 1.0 / sqrt(var) + eps;"),
    "logsm_sign": ("y[j] = (x[j] - m) - ld;", "y[j] = (x[j] - m) + ld;"),
    "logsm_log2": ("double ld = log(d);", "double ld = log2(d);"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    c = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"{name}.so")
    with open(c, "w") as f:
        f.write(text.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", c, "-o", so, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=so, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-2000:]


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = dict(zip(MUTANTS, ex.map(lambda n: _run_mutant(n, tmp), MUTANTS)))
    survivors = {n: out for n, (rc, out) in results.items() if rc == 0}
    assert not survivors, f"pins did not catch: {sorted(survivors)}"
    # a failure must be a failed assertion, not a crash of the harness
    for n, (rc, out) in results.items():
        assert rc == 1, (n, rc, out)
