"""The oracle against its pins (CPU only).  See oracle_pins.py for what each
pin checks and which passage of the pages or which piece of mathematics fixes
it."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle_pins as P  # noqa: E402
from oracle import oracle as O  # noqa: E402


@pytest.fixture(scope="module")
def orc():
    return O.default()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_arguments(orc):
    s = np.array([0.0, 1.0, 2.0])
    for k, alpha in [(0.0, 1.0), (3.0, 1.0), (-1.0, 1.0), (1.0, 0.0), (1.0, -1.0), (1.0, float("nan")),
                     (1.0, float("inf"))]:
        with pytest.raises(O.OracleError) as e:
            orc.threshold(s, k, alpha)
        assert e.value.code == O.EINVAL
    with pytest.raises(O.OracleError) as e:
        orc.threshold(np.array([], dtype=np.float64), 0.5, 1.0)
    assert e.value.code == O.EINVAL
    for bad in (float("nan"), float("inf"), -float("inf")):
        with pytest.raises(O.OracleError) as e:
            orc.threshold(np.array([0.0, bad, 1.0]), 1.0, 1.0)
        assert e.value.code == O.ENONFINITE


def test_c1_threshold_golden(orc):
    """The C1 workload's threshold, as stored by tests/golden/make_golden.py."""
    import json
    from differentiable_soft_top_amd.workloads import make_workload
    with open(os.path.join(os.path.dirname(__file__), "golden", "thresholds.json")) as f:
        gold = json.load(f)["c1"]
    s, k, alpha, _ = make_workload("c1")
    b = orc.threshold(s, k, alpha)
    assert b == pytest.approx(gold["b"], abs=1e-12)
    # and independently of the oracle's route: the definition gives mass k
    assert abs(P.mass_def(s, b, alpha) - k) <= 1e-9 * k
