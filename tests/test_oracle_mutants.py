"""Pins are sensitive: plant plausible mistakes in a copy of the oracle's C
source (a dropped term, a wrong sign, a wrong index, a transposed operand),
build each copy with gcc, and check that the pin battery rejects every one.
The committed oracle is never modified; mistakes live only in temp copies."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "softtopk_oracle.c")

MUTANTS = {
    "drop_half_prefix": ("0.5 * A[(j)] + (double)(n - 1 - (j))", "A[(j)] + (double)(n - 1 - (j))"),
    "count_off_by_one": ("(double)(n - 1 - (j))", "(double)(n - (j))"),
    "suffix_index": ("- 0.5 * B[(j) + 1] * exp", "- 0.5 * B[(j)] * exp"),
    "prefix_sign": ("A[j] = 1.0 + A[j - 1] * exp((x[j - 1] - x[j]) / alpha);",
                    "A[j] = 1.0 + A[j - 1] * exp((x[j] - x[j - 1]) / alpha);"),
    "suffix_drop_one": ("B[j] = 1.0 + B[j + 1] * exp((x[j] - x[j + 1]) / alpha);",
                        "B[j] = B[j + 1] * exp((x[j] - x[j + 1]) / alpha);"),
    "gap_transposed": ("return x_hi + alpha * log((c + r) / B);", "return x_hi + alpha * log((c + r) / A);"),
    "gap_sign": ("return x_lo - alpha * log((-c + r) / A);", "return x_lo + alpha * log((-c + r) / A);"),
    "gap_log_form": ("0.5 * alpha * log(A / B)", "0.5 * alpha * log(B / A)"),
    "below_all_operand": ("b = x[0] + alpha * log(2.0 * ((double)n - k) / B[0]);",
                          "b = x[0] + alpha * log(2.0 * ((double)n - k) / A[0]);"),
    "above_all_factor": ("b = x[n - 1] - alpha * log(2.0 * k / A[n - 1]);",
                         "b = x[n - 1] - alpha * log(k / A[n - 1]);"),
    "cdf_sign": ("return 1.0 - 0.5 * exp(-x);", "return 1.0 - 0.5 * exp(x);"),
    "p_direction": ("p_out[i] = laplace_cdf((s[i] - b) / alpha);", "p_out[i] = laplace_cdf((b - s[i]) / alpha);"),
    "vjp_drop_ratio": ("grad_out[i] = (d / alpha) * (g[i] - ratio);", "grad_out[i] = (d / alpha) * g[i];"),
    "vjp_scale": ("grad_out[i] = (d / alpha) * (g[i] - ratio);", "grad_out[i] = d * (g[i] - ratio);"),
    "mass_direction": ("m += laplace_cdf((s[i] - b) / alpha);", "m += laplace_cdf((b - s[i]) / alpha);"),
    "mass_overwrite": ("m += laplace_cdf((s[i] - b) / alpha);", "m = laplace_cdf((s[i] - b) / alpha);"),
    "mass_skip_first": ("for (int64_t i = 0; i < n; ++i)\n        m +=", "for (int64_t i = 1; i < n; ++i)\n        m +="),
    "mass_scale": ("m += laplace_cdf((s[i] - b) / alpha);", "m += laplace_cdf((s[i] - b) * alpha);"),
    "dftopk_kth_only": ("*b_out = 0.5 * (x[n - kk] + x[n - kk - 1]);", "*b_out = 0.5 * (x[n - kk] + x[n - kk]);"),
    "dftopk_smallest": ("*b_out = 0.5 * (x[n - kk] + x[n - kk - 1]);", "*b_out = 0.5 * (x[kk] + x[kk - 1]);"),
    "dftopk_shifted_rank": ("*b_out = 0.5 * (x[n - kk] + x[n - kk - 1]);",
                            "*b_out = 0.5 * (x[n - kk - 1] + x[n - kk - 1 > 0 ? n - kk - 2 : 0]);"),
    "dftopk_p_direction": ("p_out[j] = laplace_cdf((s[j] - b) / alpha);", "p_out[j] = laplace_cdf((b - s[j]) / alpha);"),
    "locate_strict": ("if (BREAK_MASS(mid) >= k)\n                lo = mid;", "if (BREAK_MASS(mid) < k)\n                lo = mid;"),
}

RUNNER = r"""
import sys
sys.path.insert(0, %(tests)r)
sys.path.insert(0, %(root)r)
from oracle.oracle import Oracle
import oracle_pins as P
orc = Oracle(sys.argv[1])
order = [P.pin_mass, P.pin_dftopk, P.pin_two_point_midpoint, P.pin_all_equal, P.pin_symmetric_sets, P.pin_logsumexp_extremes,
         P.pin_zero_temperature, P.pin_large_temperature, P.pin_mass_and_order, P.pin_invariances,
         P.pin_vjp, P.pin_bisection]
for pin in order:
    try:
        pin(orc)
    except Exception as e:
        print("caught by", pin.__name__, type(e).__name__)
        sys.exit(3)
print("survived")
sys.exit(0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation site vanished: %s" % name
    mutated = text.replace(old, new, 1)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = tmp_path / "mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(lib), str(src), "-lm"], check=True)
    runner = tmp_path / "run.py"
    runner.write_text(RUNNER % {"tests": HERE, "root": ROOT})
    r = subprocess.run([sys.executable, str(runner), str(lib)], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "mutant %s survived every pin:\n%s" % (name, r.stdout + r.stderr)
