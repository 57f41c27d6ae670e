"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars (for fp32 inputs): |b_gpu - b_ref| <= 1e-5 * alpha, max|p_gpu - p_ref| <=
1e-5, |sum p - k| <= 1e-3, backward rel-L2 <= 1e-4.  "sum p" is measured two
ways: M_p, the fp64 sum of the GPU's fp32 p, and M_b, the oracle's fp64 mass
at the GPU's b.  M_b carries the 1e-3 bar everywhere; M_p carries it on top of
the oracle's own fp32-rounding floor (the fp64 sum of the oracle's p rounded
to fp32), which on the clustered workload alone exceeds 1e-3.

Small cases are compared element by element; the full-size workloads (the
sizes the benchmark times, same launch configuration) on sampled indices
against the oracle's threshold stored in tests/golden/thresholds.json plus
properties that hold at any size.
"""
import hashlib
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import differentiable_soft_top_amd as stk  # noqa: E402
from differentiable_soft_top_amd import _lib  # noqa: E402
from differentiable_soft_top_amd.workloads import draw_grad, draw_scores, make_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "thresholds.json")) as _f:
    GOLD = json.load(_f)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    return torch.device("cuda:0")


def params(**kw):
    p = stk.default_params()
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def run(dev, s_np, k, alpha, g_np=None, prm=None):
    s = torch.from_numpy(s_np).to(dev)
    p, b, st = stk.forward(s, k, alpha, prm, want_stats=True)
    out = {"p": p.cpu().numpy().astype(np.float64), "b": float(b.item()), "stats": st}
    if g_np is not None:
        g = torch.from_numpy(g_np).to(dev)
        out["grad"] = stk.backward(g, s, alpha, b).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    return out


def check_full(res, s_np, k, alpha, g_np=None, mass_floor=0.0):
    p_ref, b_ref = O.forward(s_np, k, alpha)
    b = res["b"]
    assert abs(b - b_ref) <= 1e-5 * alpha, (b, b_ref, (b - b_ref) / alpha)
    assert np.max(np.abs(res["p"] - p_ref)) <= 1e-5
    m_b = O.mass(s_np, b, alpha)
    assert abs(m_b - k) <= 1e-3, m_b - k
    floor = abs(float(np.sum(p_ref.astype(np.float32).astype(np.float64))) - k)
    assert abs(float(np.sum(res["p"])) - k) <= 1e-3 + max(floor, mass_floor)
    if g_np is not None:
        grad_ref = O.backward(g_np, s_np, alpha, b_ref)
        err = np.linalg.norm(res["grad"] - grad_ref)
        ref = np.linalg.norm(grad_ref)
        # n = 1, or every d_i below the fp32 range: the gradient is 0
        assert np.all(np.isfinite(res["grad"]))
        assert err <= 1e-4 * ref or err <= 1e-30, (err, ref)
    return b_ref


# --------------------------------------------------------------------------
# element-by-element parity at sizes the oracle finishes in seconds; every
# size spans several pass-1 work-groups and band buckets and ends ragged
# --------------------------------------------------------------------------
SMALL = [
    ("c1", None),            # the 4096-score workload itself
    ("c2", 100_003),
    ("c3", 200_001),
    ("c4", 300_007),
    ("c2", 1_000_000),
    ("c3", 1_000_001),
]


ROUTES = {"auto": None, "steps": _lib.BAND_REFINE_STEPS, "direct": _lib.BAND_DIRECT, "buckets": _lib.BAND_BUCKETS}


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("name,n", SMALL, ids=["%s-%s" % (a, b) for a, b in SMALL])
def test_small_parity(dev, name, n, route):
    """Every band route on the same inputs: the automatic one refines the
    band on one work-group at these sizes; "steps" forces the refinement's
    step kernels (the route of larger bands); "direct" sorts the band whole
    and "buckets" sorts it by value buckets (the sorted routes, which a
    refinement that does not end falls back to).  (c1 is short enough for
    the one-kernel route by default, so the bracketed route is forced.)"""
    s_np, k, alpha, w = make_workload(name, n=n)
    g_np = draw_grad(s_np.size, w.seed)
    prm = params(force_path=_lib.PATH_BRACKET)
    if ROUTES[route] is not None:
        prm.band_route = ROUTES[route]
    res = run(dev, s_np, k, alpha, g_np, prm)
    b_ref = check_full(res, s_np, k, alpha, g_np)
    st = res["stats"]
    assert st["path"] == _lib.PATH_BRACKET, st
    want = ROUTES[route] if ROUTES[route] is not None else _lib.BAND_REFINE
    assert st["band_route"] == want, st
    if want in (_lib.BAND_REFINE, _lib.BAND_REFINE_STEPS):
        # the refinement ends on the exact closed form: fp64 rounding apart
        assert abs(res["b"] - b_ref) <= 1e-9 * alpha, (res["b"], b_ref)
        assert 1 <= st["refine_passes"] <= 8, st
    else:
        assert st["refine_passes"] == 0, st


def test_direct_band_overflow_falls_back_to_buckets(dev):
    """A band forced onto the whole-band sort but larger than it (about 11,700
    scores here) is bucketed instead, in the same round, without a new pass.
    The automatic route refines the same band with the step kernels (its
    expected size is past the one-work-group form) and reaches the same b."""
    s_np, k, alpha, w = make_workload("c4", n=3_000_007)
    res = run(dev, s_np, k, alpha, None, params(band_route=_lib.BAND_DIRECT))
    st = res["stats"]
    assert st["n_band"] > 8192 and st["rounds"] == 1, st
    assert st["path"] == _lib.PATH_BRACKET and st["band_route"] == _lib.BAND_BUCKETS, st
    check_full(res, s_np, k, alpha)
    auto = run(dev, s_np, k, alpha)
    assert auto["stats"]["band_route"] == _lib.BAND_REFINE_STEPS, auto["stats"]
    assert abs(auto["b"] - res["b"]) <= 1e-9 * alpha, (auto["b"], res["b"])


@pytest.mark.parametrize("k", [1.0, 199_999.0])
def test_refine_chain_resumes(dev, k):
    """An open bracket (k near 0 or n with 1024 samples leaves one end at
    infinity): the step kernels start at the finite end, far from b, and
    need more passes than a chain holds; each chain that runs out resumes
    where it stopped, and the end is the exact root."""
    n = 200_000
    s_np = draw_scores("normal", n, seed=21)
    alpha = 0.05
    g_np = draw_grad(n, 21)
    res = run(dev, s_np, k, alpha, g_np, params(samples=1024, band_route=_lib.BAND_REFINE_STEPS))
    b_ref = check_full(res, s_np, k, alpha, g_np)
    st = res["stats"]
    assert st["band_route"] == _lib.BAND_REFINE_STEPS, st
    assert not (np.isfinite(st["a_left"]) and np.isfinite(st["a_right"])), st
    assert st["refine_passes"] > 8, st  # more than the longest chain
    assert abs(res["b"] - b_ref) <= 1e-9 * alpha


@pytest.mark.parametrize("name,n,cap", [("c2", 100_003, 16), ("c4", 300_007, 256), ("c3", 200_001, 256),
                                        ("c5", 100_000, 1000), ("c2", 8_193, 16)])
def test_band_overflow_refines_every_score(dev, name, n, cap):
    """A band larger than its buffer: the refinement runs over every score
    (no tails, no bracket) from the bracket's middle and ends on the exact
    root, in the same round."""
    s_np, k, alpha, w = make_workload(name, n=n)
    g_np = draw_grad(s_np.size, w.seed)
    res = run(dev, s_np, k, alpha, g_np, params(band_capacity=cap, force_path=_lib.PATH_BRACKET))
    b_ref = check_full(res, s_np, k, alpha, g_np)
    st = res["stats"]
    assert st["path"] == _lib.PATH_ALL_SCORES and st["rounds"] == 1, st
    assert st["reject_mask"] & _lib.REJECT_OVERFLOW and st["band_route"] == _lib.BAND_REFINE_STEPS, st
    assert abs(res["b"] - b_ref) <= 1e-9 * alpha, (res["b"], b_ref)


def test_clustered_small(dev):
    """60% of the scores tied exactly at the threshold.  At this size the tied
    band still fits its buffer, so the certified route handles it (refined,
    and sorted, where the cluster lands in one all-equal bucket); with a
    small band capacity the refinement runs over every score, and the sorted
    route takes the full sort.  All must match the oracle."""
    s_np, k, alpha, w = make_workload("c5", n=100_000)
    g_np = draw_grad(s_np.size, w.seed)
    for route in (0, _lib.BAND_BUCKETS):
        res = run(dev, s_np, k, alpha, g_np, params(band_route=route))
        check_full(res, s_np, k, alpha, g_np)
        assert res["stats"]["path"] == _lib.PATH_BRACKET, res["stats"]
    res = run(dev, s_np, k, alpha, g_np, params(band_capacity=1000))
    check_full(res, s_np, k, alpha, g_np)
    assert res["stats"]["path"] == _lib.PATH_ALL_SCORES, res["stats"]
    res = run(dev, s_np, k, alpha, g_np, params(band_capacity=1000, band_route=_lib.BAND_BUCKETS))
    check_full(res, s_np, k, alpha, g_np)
    assert res["stats"]["path"] == _lib.PATH_FULLSORT, res["stats"]
    assert res["stats"]["reject_mask"] & _lib.REJECT_OVERFLOW


def test_overflow_expected_from_the_last_call(dev):
    """After a call whose band overflowed, the next call with the same n, k,
    alpha and band capacity only counts its band in pass-1 and refines every
    score, on a wider grid (so its sums round in another order): the same b
    to 1e-9 alpha, and the same exact band count.  A vector
    whose band fits, called with that shape, is still solved exactly (every
    score refined, the band count exact and within the capacity), and the
    call after it keeps its band again."""
    cap = 8000
    s_a, k, alpha, w = make_workload("c5", n=100_000)  # 60% tied: the band holds them
    g_np = draw_grad(s_a.size, w.seed)
    first = run(dev, s_a, k, alpha, g_np, params(band_capacity=cap))
    second = run(dev, s_a, k, alpha, g_np, params(band_capacity=cap))
    for res in (first, second):
        check_full(res, s_a, k, alpha, g_np)
        assert res["stats"]["path"] == _lib.PATH_ALL_SCORES, res["stats"]
        assert res["stats"]["n_band"] > cap, res["stats"]
    assert abs(second["b"] - first["b"]) <= 1e-9 * alpha and second["stats"]["n_band"] == first["stats"]["n_band"]
    s_b = np.random.default_rng(5).standard_normal(s_a.size).astype(np.float32)
    counted = run(dev, s_b, k, alpha, g_np, params(band_capacity=cap))
    check_full(counted, s_b, k, alpha, g_np)
    st = counted["stats"]
    assert st["path"] == _lib.PATH_ALL_SCORES and 0 < st["n_band"] <= cap, st
    kept = run(dev, s_b, k, alpha, g_np, params(band_capacity=cap))
    check_full(kept, s_b, k, alpha, g_np)
    assert kept["stats"]["path"] == _lib.PATH_BRACKET and kept["stats"]["n_band"] == st["n_band"], kept["stats"]


@pytest.mark.parametrize("name,n", [("c1", None), ("c2", 100_003), ("c4", 300_007), ("c3", 65_537)])
def test_forced_full_sort_matches(dev, name, n):
    s_np, k, alpha, w = make_workload(name, n=n)
    g_np = draw_grad(s_np.size, w.seed)
    res = run(dev, s_np, k, alpha, g_np, params(force_path=_lib.PATH_FULLSORT))
    assert res["stats"]["path"] == _lib.PATH_FULLSORT
    check_full(res, s_np, k, alpha, g_np)


@pytest.mark.parametrize("where,alpha", [("above", 1e-3), ("below", 1e-3), ("pinned", 1e-3), ("pinned", 1e-4)])
def test_tied_cluster_splits_the_bracket(dev, where, alpha):
    """600,000 of 10^6 scores tied at T = 0.5.  "above" / "below": b lies
    0.02 alpha above / below T (hundreds of fp32 ulps); the sampled bracket
    around b holds the cluster, so the band overflows; the bracket is then
    split at T, the cluster lands in one tail, and that round certifies
    without the full sort.  "pinned": k is set (by the oracle's M) between
    M(T+) and M(T), T+ the next float above T, so b lies strictly inside
    (T, T+): both sides reject and the closed form in the gap right of T
    gives b (at alpha 1e-3 and at the clustered workload's 1e-4).  With no
    widening rounds allowed, the full sort gives the same b.  (The split
    belongs to the sorted band routes, forced here: by default an overflowing
    band is refined over every score, which must give the same b too.)"""
    n, n_tie = 1_000_000, 600_000
    rng = np.random.default_rng(31)
    s_np = rng.standard_normal(n).astype(np.float32)
    s_np[:n_tie] = np.float32(0.5)
    s_np = s_np[rng.permutation(n)]
    n_above = float(np.count_nonzero(s_np > 0.5))
    t_up = float(np.nextafter(np.float32(0.5), np.float32(1.0)))
    if where == "pinned":
        k = 0.5 * (O.mass(s_np, 0.5, alpha) + O.mass(s_np, t_up, alpha))
    else:
        k = n_above + (0.49 if where == "above" else 0.51) * n_tie
    g_np = rng.standard_normal(n).astype(np.float32)
    res = run(dev, s_np, k, alpha, g_np, params(band_route=_lib.BAND_BUCKETS))
    check_full(res, s_np, k, alpha, g_np)
    st = res["stats"]
    assert st["path"] == _lib.PATH_WIDENED and st["reject_mask"] & _lib.REJECT_OVERFLOW, st
    if where == "above":
        assert st["a_left"] > 0.5, st
    elif where == "below":
        assert st["a_right"] == np.float32(0.5), st
    else:
        both = _lib.REJECT_LOW | _lib.REJECT_HIGH
        assert st["reject_mask"] & both == both and 0.5 < res["b"] < t_up, st
    full = run(dev, s_np, k, alpha, None, params(max_widen=0, band_route=_lib.BAND_BUCKETS))
    assert full["stats"]["path"] == _lib.PATH_FULLSORT, full["stats"]
    assert abs(full["b"] - res["b"]) <= 2e-5 * alpha
    refined = run(dev, s_np, k, alpha, g_np)
    check_full(refined, s_np, k, alpha, g_np)
    assert refined["stats"]["path"] == _lib.PATH_ALL_SCORES, refined["stats"]
    assert abs(refined["b"] - full["b"]) <= 2e-5 * alpha


@pytest.mark.parametrize("k", [5000.0, 5000.25, 4000.0])
def test_root_in_a_wide_gap(dev, k):
    """Scores 0.74 apart with alpha = 1e-3: b lies in a gap of 740 alpha, so at
    a split near its middle both sums are about e^-370 and their product
    leaves the normal fp64 range; the steps form the discriminant without
    it.  k = 5000 puts b exactly in the middle of a gap (d = 0 there)."""
    n = 10_000
    s_np = (np.random.default_rng(17).permutation(n) * 0.74).astype(np.float32)
    g_np = np.random.default_rng(18).standard_normal(n).astype(np.float32)
    for route in (0, _lib.BAND_REFINE_STEPS):
        res = run(dev, s_np, k, 1e-3, g_np, params(band_route=route))
        check_full(res, s_np, k, 1e-3, g_np)


@pytest.mark.parametrize("k", [2000.25, 10_000.0, 17_000.5])
def test_evenly_spaced_scores_at_small_alpha(dev, k):
    """A vector of the integers 0..19999 (shuffled) with alpha a hundredth of
    their spacing: the band's model steps cross about one score per pass, so
    a refinement that starts far from b may not end within its passes and
    the band is sorted instead.  Every route gives the oracle's b."""
    n, alpha = 20_000, 0.01
    s_np = np.random.default_rng(23).permutation(n).astype(np.float32)
    g_np = np.random.default_rng(24).standard_normal(n).astype(np.float32)
    for route in (0, _lib.BAND_REFINE_STEPS, _lib.BAND_BUCKETS):
        res = run(dev, s_np, k, alpha, g_np, params(band_route=route))
        check_full(res, s_np, k, alpha, g_np)


def test_route_independence(dev):
    """Different Philox seeds, a too-narrow bracket (forcing rejections and
    widening), an overfull band and the forced full sort all give the same b."""
    s_np, k, alpha, _ = make_workload("c2", n=200_000)
    _, b_ref = O.forward(s_np, k, alpha)
    bs = {}
    for tag, prm in [("seed1", params(seed=1)), ("seed2", params(seed=0xABCDEF)),
                     ("narrow", params(z=0.05, max_widen=4)),
                     ("overflow", params(band_capacity=16)),
                     ("overflow_sorted", params(band_capacity=16, band_route=_lib.BAND_BUCKETS)),
                     ("narrow_sorted", params(z=0.05, max_widen=4, band_route=_lib.BAND_DIRECT)),
                     ("full", params(force_path=_lib.PATH_FULLSORT))]:
        res = run(dev, s_np, k, alpha, None, prm)
        bs[tag] = (res["b"], res["stats"])
        assert abs(res["b"] - b_ref) <= 1e-5 * alpha, (tag, res["b"], b_ref)
    assert bs["overflow"][1]["path"] == _lib.PATH_ALL_SCORES
    assert bs["overflow_sorted"][1]["path"] == _lib.PATH_FULLSORT
    for tag in ("overflow", "overflow_sorted"):
        assert bs[tag][1]["reject_mask"] & _lib.REJECT_OVERFLOW
    assert bs["full"][1]["path"] == _lib.PATH_FULLSORT


def test_narrow_bracket_widens(dev):
    """With z tiny, the first bracket usually misses b; the certificate
    rejects it and the widened bracket (or the full sort) still gives b."""
    hits = 0
    for seed in range(6):
        s_np, k, alpha, _ = make_workload("c2", n=100_000, seed=seed)
        res = run(dev, s_np, k, alpha, None, params(z=0.02, max_widen=6, seed=seed + 11))
        _, b_ref = O.forward(s_np, k, alpha)
        assert abs(res["b"] - b_ref) <= 1e-5 * alpha
        st = res["stats"]
        if st["reject_mask"] & (_lib.REJECT_LOW | _lib.REJECT_HIGH):
            hits += 1
            # (a widened bracket can be open-ended and overflow the band,
            # which then refines every score)
            assert st["path"] in (_lib.PATH_WIDENED, _lib.PATH_FULLSORT, _lib.PATH_ALL_SCORES)
            assert st["rounds"] >= 2 or st["path"] == _lib.PATH_FULLSORT
    assert hits >= 1


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------
EDGE = [
    ("n1_klow", np.array([0.7], np.float32), 0.3, 1.0),
    ("n1_khigh", np.array([-2.0], np.float32), 0.9, 0.5),
    ("n2_mid", np.array([1.0, 3.0], np.float32), 1.0, 0.25),
    ("n3", np.array([0.0, 1.0, 2.0], np.float32), 1.5, 1.0),
    ("n5_ragged", np.array([5.0, -1.0, 2.5, 2.5, 0.0], np.float32), 2.2, 0.3),
    ("n7_ties", np.array([1, 1, 1, 2, 2, 3, 3], np.float32), 3.0, 0.01),
    ("zeros_signed", np.array([0.0, -0.0, 0.0, -0.0, 1.0, -1.0], np.float32), 3.0, 0.5),
]


@pytest.mark.parametrize("route", ["auto", "bracket"])
@pytest.mark.parametrize("tag,s_np,k,alpha", EDGE, ids=[e[0] for e in EDGE])
def test_tiny_inputs(dev, tag, s_np, k, alpha, route):
    g_np = np.linspace(-1, 1, s_np.size).astype(np.float32)
    prm = params(force_path=_lib.PATH_BRACKET) if route == "bracket" else None
    res = run(dev, s_np, k, alpha, g_np, prm)
    check_full(res, s_np, k, alpha, g_np)
    want = _lib.PATH_BRACKET if route == "bracket" else _lib.PATH_SINGLE
    assert res["stats"]["path"] == want, res["stats"]


@pytest.mark.parametrize("n", [2, 63, 64, 65, 300, 1000, 1024, 1025, 2000, 4096, 8191, 8192, 8193])
def test_single_kernel_route(dev, n):
    """Vectors of at most 8192 scores take the one-kernel route by default
    (the whole vector sorted in registers and solved exactly, then the fp64
    mass published); longer ones the bracketed route.  Both match the oracle
    and agree with the bracketed route forced at the same size."""
    rng = np.random.default_rng(n)
    s_np = rng.standard_normal(n).astype(np.float32)
    s_np[: n // 3] = np.round(s_np[: n // 3] * 4.0) / 4.0  # some ties
    s_np = s_np[rng.permutation(n)]
    g_np = rng.standard_normal(n).astype(np.float32)
    for k in (0.5, n / 10.0, n - 0.25):
        res = run(dev, s_np, k, 0.05, g_np)
        check_full(res, s_np, k, 0.05, g_np)
        st = res["stats"]
        assert st["path"] == (_lib.PATH_SINGLE if n <= 8192 else _lib.PATH_BRACKET), st
        assert abs(st["mass"] - k) <= 1e-3, st
        assert st["b"] == res["b"]
        forced = run(dev, s_np, k, 0.05, g_np, params(force_path=_lib.PATH_BRACKET))
        assert forced["stats"]["path"] in (_lib.PATH_BRACKET, _lib.PATH_WIDENED, _lib.PATH_FULLSORT)
        assert abs(forced["b"] - res["b"]) <= 2e-5 * 0.05


def test_single_kernel_route_rejects_nonfinite_and_checks_mass(dev):
    s_np = np.random.default_rng(5).standard_normal(3000).astype(np.float32)
    for bad in (np.nan, np.inf, -np.inf):
        t = s_np.copy()
        t[2999] = bad
        with pytest.raises(stk.SoftTopKError) as e:
            stk.forward(torch.from_numpy(t).to(dev), 100.0, 0.1)
        assert e.value.code == _lib.ENONFINITE
    # the mass check on request, and the stats without it
    res = run(dev, s_np, 100.0, 0.1, None, params(verify_mass=1))
    assert res["stats"]["path"] == _lib.PATH_SINGLE and abs(res["stats"]["mass"] - 100.0) <= 1e-3
    check_full(res, s_np, 100.0, 0.1)


@pytest.mark.parametrize("case", ["equal", "sorted", "reversed", "k_tiny", "k_near_n", "alpha_huge",
                                  "alpha_tiny", "negative", "bimodal", "k_half", "saturated"])
def test_structured_inputs(dev, case):
    rng = np.random.default_rng(99)
    n = 50_021
    alpha = 0.05
    if case == "equal":
        s = np.full(n, 0.25, np.float32)
        k = 1234.5
    elif case == "sorted":
        s = draw_scores("sorted_normal", n, 3)
        k = 500.0
    elif case == "reversed":
        s = np.ascontiguousarray(draw_scores("sorted_normal", n, 4)[::-1])
        k = 500.0
    elif case == "k_tiny":
        s = rng.standard_normal(n).astype(np.float32)
        k = 1e-3
    elif case == "k_near_n":
        s = rng.standard_normal(n).astype(np.float32)
        k = n - 1e-3
    elif case == "alpha_huge":
        s = rng.standard_normal(n).astype(np.float32)
        k, alpha = 100.0, 1e3
    elif case == "alpha_tiny":
        s = rng.standard_normal(n).astype(np.float32)
        k, alpha = 100.0, 1e-6
    elif case == "negative":
        s = (rng.standard_normal(n) - 50.0).astype(np.float32)
        k = 2000.0
    elif case == "saturated":
        # b below every score and one score well apart from the rest: its
        # density dominates D, so its gradient g_i - G/D nearly cancels
        s = rng.standard_normal(n).astype(np.float32)
        s[np.argmin(s)] -= 1.0
        k = n - 0.5
    elif case == "bimodal":
        s = np.concatenate([rng.normal(-3, 0.1, n // 2), rng.normal(3, 0.1, n - n // 2)]).astype(np.float32)
        s = s[rng.permutation(n)]
        k = n / 2
    else:
        s = rng.standard_normal(n).astype(np.float32)
        k = n / 2
    g = rng.standard_normal(n).astype(np.float32)
    res = run(dev, s, k, alpha, g)
    check_full(res, s, k, alpha, g)


def test_unaligned_pointers(dev):
    """Scores / outputs not 16-byte aligned take the scalar-load kernels."""
    s_np, k, alpha, w = make_workload("c2", n=100_003)
    g_np = draw_grad(s_np.size, w.seed)
    base = torch.from_numpy(np.concatenate([[0.0], s_np]).astype(np.float32)).to(dev)
    s = base[1:]
    assert s.data_ptr() % 16 != 0
    gbase = torch.from_numpy(np.concatenate([[0.0], g_np]).astype(np.float32)).to(dev)
    g = gbase[1:]
    p, b = stk.forward(s, k, alpha)
    grad = stk.backward(g, s, alpha, b)
    res = {"p": p.cpu().numpy().astype(np.float64), "b": float(b.item()),
           "grad": grad.cpu().numpy().astype(np.float64)}
    check_full(res, s_np, k, alpha, g_np)


def test_nonfinite_is_rejected(dev):
    s_np = np.random.default_rng(1).standard_normal(10_000).astype(np.float32)
    for bad in (np.nan, np.inf, -np.inf):
        t = s_np.copy()
        t[1234] = bad
        with pytest.raises(stk.SoftTopKError) as e:
            stk.forward(torch.from_numpy(t).to(dev), 100.0, 0.1)
        assert e.value.code == _lib.ENONFINITE
        with pytest.raises(stk.SoftTopKError) as e:
            stk.forward(torch.from_numpy(t).to(dev), 100.0, 0.1, params(force_path=_lib.PATH_FULLSORT))
        assert e.value.code == _lib.ENONFINITE


def test_invalid_arguments_raise(dev):
    s = torch.zeros(10, device=dev)
    for k, alpha in [(0.0, 1.0), (10.0, 1.0), (1.0, 0.0)]:
        with pytest.raises(stk.SoftTopKError) as e:
            stk.forward(s, k, alpha)
        assert e.value.code == _lib.EINVAL


def test_deterministic(dev):
    s_np, k, alpha, _ = make_workload("c2", n=500_000)
    s = torch.from_numpy(s_np).to(dev)
    p1, b1 = stk.forward(s, k, alpha)
    p2, b2 = stk.forward(s, k, alpha)
    assert float(b1.item()) == float(b2.item())
    assert torch.equal(p1, p2)


def test_deterministic_large_buckets(dev):
    # ~40k band scores in 512 buckets: the order inside a bucket depends on
    # atomic reservations, so this checks that the bucket sums do not
    s_np, k, alpha, _ = make_workload("c3")
    s = torch.from_numpy(s_np).to(dev)
    runs = [stk.forward(s, k, alpha) for _ in range(3)]
    b0 = float(runs[0][1].item())
    for p, b in runs[1:]:
        assert float(b.item()) == b0
        assert torch.equal(p, runs[0][0])


def test_autograd_and_side_stream(dev):
    s_np, k, alpha, w = make_workload("c1")
    g_np = draw_grad(s_np.size, w.seed)
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        s = torch.from_numpy(s_np).to(dev).requires_grad_(True)
        p, b = stk.soft_topk(s, k, alpha)
        (p * torch.from_numpy(g_np).to(dev)).sum().backward()
    side.synchronize()
    _, b_ref = O.forward(s_np, k, alpha)
    grad_ref = O.backward(g_np, s_np, alpha, b_ref)
    grad = s.grad.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(grad - grad_ref) / np.linalg.norm(grad_ref) <= 1e-4
    assert abs(float(grad.sum())) <= 1e-3 * np.abs(grad).sum()


# --------------------------------------------------------------------------
# the sampler: device Philox draws against the published definition
# --------------------------------------------------------------------------
def _philox_ref(counter, key):
    M0, M1, W0, W1 = 0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85
    c = list(counter)
    k0, k1 = key
    for _ in range(10):
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k0, p1 & 0xFFFFFFFF, (p0 >> 32) ^ c[3] ^ k1, p0 & 0xFFFFFFFF]
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return c


def test_philox_reference_known_answers():
    # Random123 known-answer vectors for Philox4x32-10
    assert _philox_ref([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert _philox_ref([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]


def test_sampler_matches_philox_definition(dev):
    n = 123_457
    s_np = np.random.default_rng(5).standard_normal(n).astype(np.float32)
    alpha = 0.25
    seed = 0x0123456789ABCDEF
    m = 2048
    s = torch.from_numpy(s_np).to(dev)
    out = torch.empty(m, dtype=torch.float32, device=dev)
    lib = _lib.load()
    import ctypes
    rc = lib.soft_topk_debug_sample(ctypes.c_void_p(s.data_ptr()), n, alpha, seed, m,
                                    ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    _lib.check(rc, "debug_sample")
    y = out.cpu().numpy()
    k0, k1 = seed & 0xFFFFFFFF, seed >> 32
    for j in range(m):
        w = _philox_ref([j, 0, 0, 0], [k0, k1])
        idx = ((w[1] << 32 | w[0]) * n) >> 64
        u = (w[2] + 0.5) / 2.0 ** 32
        e = np.log(2 * u) if u < 0.5 else -np.log(2 * (1 - u))
        ref = np.float32(float(s_np[idx]) + float(np.float32(alpha)) * e)
        assert abs(float(y[j]) - float(ref)) <= 2 * abs(float(np.spacing(ref))), (j, y[j], ref)


@pytest.mark.parametrize("name,n,kfrac,prm", [
    ("c2", 100_003, None, {}),
    ("c3", 200_001, None, {"seed": 77}),
    ("c4", 300_007, None, {"samples": 4096, "z": 3.0}),
    ("c2", 100_003, 0.5, {}),
    ("c2", 50_001, 0.999, {"samples": 1024, "z": 6.0}),
], ids=["c2", "c3-seed", "c4-m4096", "c2-median", "c2-tail-m1024"])
def test_bracket_is_the_exact_order_statistics(dev, name, n, kfrac, prm):
    """The first round's bracket ends are the order statistics of the m
    kernel-noised samples at the binomial ranks, exactly: the device selects
    them digit by digit, the test sorts the same samples on the host.  The
    median case passes over 8192 candidates to the selection (16 keys per
    thread)."""
    import ctypes
    s_np, k, alpha, _ = make_workload(name, n=n)
    if kfrac is not None:
        k = kfrac * s_np.size
    p = params(**prm)
    res = run(dev, s_np, k, alpha, None, p)
    st = res["stats"]
    assert st["rounds"] == 1 and st["path"] == _lib.PATH_BRACKET, st
    m = p.samples
    s = torch.from_numpy(s_np).to(dev)
    out = torch.empty(m, dtype=torch.float32, device=dev)
    lib = _lib.load()
    rc = lib.soft_topk_debug_sample(ctypes.c_void_p(s.data_ptr()), s_np.size, alpha, p.seed, m,
                                    ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    _lib.check(rc, "debug_sample")
    y = np.sort(out.cpu().numpy())
    rl, rr = _lib.bracket_ranks(m, 1.0 - k / s_np.size, p.z)
    want_l = -np.inf if rl < 1 else float(y[rl - 1])
    want_r = np.inf if rr > m else float(y[rr - 1])
    assert st["a_left"] == want_l and st["a_right"] == want_r, (st["a_left"], want_l, st["a_right"], want_r)


# --------------------------------------------------------------------------
# saturated-score segments (from 2^22 scores on): the VJP reads the
# emission's record of the scores near b instead of the scores
# --------------------------------------------------------------------------
SEG_N = (1 << 24) + 4099  # whole tiles plus a ragged end


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("order,kfrac", [("random", None), ("sorted", None), ("random", 0.5), ("sorted", 0.5)])
def test_segments_match_oracle_and_score_path(dev, order, kfrac):
    """c4's law (U(0,1), alpha = 1e-3) at 2^24 + 4099 scores: most segments
    hold few listed scores; with k = n/2 many scores also lie far beyond the
    right end (p = 1 without reading them).  Sorted, the segments are all
    far-left (sparse, none listed), all listed (dense) or all far-right
    (sparse, p = 1).  Element-wise parity with the oracle, and the backward
    through the forward's record equals the score-reading backward: each
    element is the same fp32 product of the same d and g with G/D, which the
    two sum over different work-group splits (fp64, so G/D may move by an
    fp32 ulp); a zero is +0 where a record served it, and the same +-0 where
    the segment was read from the scores."""
    s_np, k, alpha, w = make_workload("c4", n=SEG_N)
    if kfrac is not None:
        k = kfrac * s_np.size
    if order == "sorted":
        s_np = np.sort(s_np)
    g_np = draw_grad(s_np.size, w.seed)
    s = torch.from_numpy(s_np).to(dev)
    g = torch.from_numpy(g_np).to(dev)
    p, b, st, ws = stk.forward(s, k, alpha, want_stats=True, want_workspace=True)
    assert st["path"] == _lib.PATH_BRACKET, st
    g_seg = stk.backward(g, s, alpha, b, fwd_workspace=ws)
    g_dense = stk.backward(g, s, alpha, b)
    torch.cuda.synchronize()
    res = {"p": p.cpu().numpy().astype(np.float64), "b": float(b.item()), "stats": st,
           "grad": g_seg.cpu().numpy().astype(np.float64)}
    check_full(res, s_np, k, alpha, g_np)
    gs, gd = g_seg.cpu().numpy(), g_dense.cpu().numpy()
    nz = gd != 0
    _assert_score_path_equal(gs, gd, g_np, alpha)
    bz = _bits(gs[~nz])
    assert np.all((bz == 0) | (bz == _bits(gd[~nz])))  # +0 from a record, else the same +-0


DENS_CUT = 2.0 ** -40  # densities the forward's record keeps (at least)


def _assert_score_path_equal(gs, gd, g_np, alpha):
    """The record-using gradient gs against the score-reading gd.  The record
    keeps the densities d >= 2^-40; a dropped one gives +0 where the score
    path gives (d/alpha)(g - G/D), below 2^-40/alpha * (|g| + max|g|) since
    |G/D| <= max|g|.  Elsewhere both are the same fp32 product of d, 1/alpha
    and g - G/D, where G/D may differ by an fp32 ulp (the two sum D and G
    over different work-group splits, and the dropped terms move them by at
    most n 2^-40): |G/D| <= max|g|, d/alpha <= 1/(2 alpha), plus each
    product's rounding."""
    gmax = float(np.max(np.abs(g_np)))
    assert np.all(gs[gd == 0] == 0)
    dropped = (gd != 0) & (gs == 0)
    if np.any(dropped):
        bound = DENS_CUT / alpha * (np.abs(g_np[dropped].astype(np.float64)) + gmax) * (1 + 1e-6)
        assert np.all(np.abs(gd[dropped]) <= bound)
    nz = (gd != 0) & (gs != 0)
    if not np.any(nz):
        return
    ulp_ratio = float(np.spacing(np.float32(gmax)))
    ulp_grad = float(np.spacing(np.float32(np.max(np.abs(gd)))))
    diff = np.max(np.abs(gs[nz].astype(np.float64) - gd[nz]))
    assert diff <= 2 * ulp_ratio / (2 * alpha) + 2 * ulp_grad, (diff, ulp_ratio, ulp_grad)


def test_segments_nonfinite_cotangent_and_foreign_threshold(dev):
    """A non-finite cotangent at a saturated score still enters G (as
    g * 0 = NaN), so the whole gradient is NaN, as in the score-reading path
    (the sign and payload of a NaN carry no meaning and may differ between
    the routes); a threshold other than the forward's makes the backward read
    the scores."""
    s_np, k, alpha, w = make_workload("c4", n=SEG_N)
    g_np = draw_grad(s_np.size, w.seed)
    far = np.flatnonzero(s_np < 0.5)[:3]
    g_np[far[0]] = np.inf
    g_np[far[1]] = np.nan
    s = torch.from_numpy(s_np).to(dev)
    g = torch.from_numpy(g_np).to(dev)
    p, b, ws = stk.forward(s, k, alpha, want_workspace=True)
    g_seg = stk.backward(g, s, alpha, b, fwd_workspace=ws).cpu().numpy()
    g_dense = stk.backward(g, s, alpha, b).cpu().numpy()
    assert np.all(np.isnan(g_seg))
    assert np.all(np.isnan(g_dense))
    g_np = draw_grad(s_np.size, w.seed)
    g = torch.from_numpy(g_np).to(dev)
    g_seg = stk.backward(g, s, alpha, b, fwd_workspace=ws).cpu().numpy()
    assert g_seg[far[2]] == 0.0 and np.all(np.isfinite(g_seg))
    _assert_score_path_equal(g_seg, stk.backward(g, s, alpha, b).cpu().numpy(), g_np, alpha)
    b2 = b + 1e-4  # another threshold: the record does not apply
    g_seg2 = stk.backward(g, s, alpha, b2, fwd_workspace=ws).cpu().numpy()
    g_dense2 = stk.backward(g, s, alpha, b2).cpu().numpy()
    _assert_score_path_equal(g_seg2, g_dense2, g_np, alpha)
    zero = g_dense2 == 0  # both read the scores: the same signed zeros
    assert np.array_equal(np.signbit(g_seg2[zero]), np.signbit(g_dense2[zero]))
    assert not np.array_equal(_bits(g_seg2), _bits(g_seg))


def test_c5_full_sort_fallback(dev):
    """The clustered workload on a sorted band route with no widening rounds
    allowed skips the tie split: the band overflow sends it to the full
    device radix sort, which returns the stored oracle b."""
    gold = GOLD["c5"]
    s_np, k, alpha, w = make_workload("c5")
    s = torch.from_numpy(s_np).to(dev)
    p, b, st = stk.forward(s, k, alpha, params(max_widen=0, band_route=_lib.BAND_BUCKETS), want_stats=True)
    assert st["path"] == _lib.PATH_FULLSORT and st["reject_mask"] & _lib.REJECT_OVERFLOW, st
    assert abs(float(b.item()) - gold["b"]) <= 1e-5 * alpha
    m = float(torch.sum(p.double()).item())
    assert abs(m - k) <= 1e-3 + gold["mass_p32_rounding_floor"], (m, k)


def test_forced_full_sort_at_full_size(dev):
    """c4 (1e8 scores) on the forced full-sort route: the radix sort over
    12,208 tiles (offsets scanned in chunks of 96) and the solve over 24,415
    summaries return the stored oracle b and the certified mass, and every
    p agrees with the default route's (whose every element
    test_gpu_fullsize compares with the oracle)."""
    gold = GOLD["c4"]
    s_np, k, alpha, w = make_workload("c4")
    s = torch.from_numpy(s_np).to(dev)
    p, b, st = stk.forward(s, k, alpha, params(force_path=_lib.PATH_FULLSORT), want_stats=True)
    assert st["path"] == _lib.PATH_FULLSORT, st
    b = float(b.item())
    assert abs(b - gold["b"]) <= 1e-5 * alpha, (b, gold["b"])
    assert abs(st["mass"] - k) <= 1e-3 + gold["mass_p32_rounding_floor"], st["mass"]
    p_default, b_default = stk.forward(s, k, alpha)
    assert abs(float(b_default.item()) - b) <= 1e-5 * alpha
    assert float(torch.max(torch.abs(p.double() - p_default.double())).item()) <= 1e-5


# --------------------------------------------------------------------------
# path coverage: the bracket certifies on its first round for every seed
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_certified_first_try_over_100_seeds(dev, name):
    """100 Philox seeds per workload: every forward takes the bracket route on
    its first round (no widening, no fallback) and returns the oracle's b.  At
    z = 5 a side fails with probability below 3e-7, so a failure here points
    at the sampler or the rank arithmetic, not at chance."""
    gold = GOLD[name]
    s_np, k, alpha, w = make_workload(name)
    s = torch.from_numpy(s_np).to(dev)
    rng = np.random.default_rng(12345)
    seeds = [int(x) for x in rng.integers(1, 2 ** 63, 100)]
    worst = 0.0
    for seed in seeds:
        _, b, st = stk.forward(s, k, alpha, params(seed=seed, force_path=_lib.PATH_BRACKET), want_stats=True)
        assert st["path"] == _lib.PATH_BRACKET and st["rounds"] == 1, (name, seed, st)
        worst = max(worst, abs(float(b.item()) - gold["b"]) / alpha)
    assert worst <= 1e-5, (name, worst)


# --------------------------------------------------------------------------
# full-size workloads with the certification pass waited for (a stats record
# turns it on); the benchmark's own call sequence, with every element compared
# with the oracle, is in test_gpu_fullsize.py
# --------------------------------------------------------------------------
def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_full_size_route_and_certified_mass(dev, name):
    """The route each full-size workload takes, b against the oracle's stored
    b, and the certification pass: the fp64 mass the library folds from its
    own p (stats.mass) and the oracle's mass at the GPU's b."""
    gold = GOLD[name]
    s_np, k, alpha, w = make_workload(name)
    assert _sha(s_np) == gold["sha256_scores"], "input generator drifted"
    assert k == gold["k"]
    s = torch.from_numpy(s_np).to(dev)
    p, b, st = stk.forward(s, k, alpha, params(verify_mass=1), want_stats=True)
    torch.cuda.synchronize()
    b_gpu = float(b.item())
    b_ref = gold["b"]
    assert abs(b_gpu - b_ref) <= 1e-5 * alpha, (b_gpu, b_ref, (b_gpu - b_ref) / alpha)
    # c5: the tied cluster overflows every band; the refinement then runs
    # over every score (its own tests force the tie split and the full sort)
    expect = _lib.PATH_ALL_SCORES if name == "c5" else _lib.PATH_BRACKET
    assert st["path"] == expect, st
    floor = gold["mass_p32_rounding_floor"]
    assert abs(st["mass"] - k) <= 1e-3 + floor, st
    m_p = float(torch.sum(p.double()).item())
    assert abs(m_p - k) <= 1e-3 + floor, (m_p, k)
    assert abs(O.mass(s_np, b_gpu, alpha) - k) <= 1e-3
