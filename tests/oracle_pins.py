"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, none of which re-types the oracle's own sort/scan/closed-form route.

Each check takes an ``Oracle`` object so the same battery can be run against
deliberately broken copies of the oracle (see test_oracle_mutants.py).

Sources (gist.science technical summary of "Fast LapSum: Exact Differentiable
Top-k at Million Scale"): section 2.1 defines p_i = F((r_i - b)/t) with F the
Laplace CDF and sum p_i = k, with an analytic backward; section 2.2 says the
full-sort solver replaces an iterative bisection on b; section 2.3 says the
zero-temperature limit puts b at the midpoint of the k-th and (k+1)-th order
statistics.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np
from scipy.special import logsumexp


# --------------------------------------------------------------------------
# independent reference pieces (definition-level, no sort, no recurrences)
# --------------------------------------------------------------------------
def lap_cdf(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    neg = x <= 0
    out[neg] = 0.5 * np.exp(x[neg])
    out[~neg] = 1.0 - 0.5 * np.exp(-x[~neg])
    return out


def mass_def(s, b, alpha):
    return float(np.sum(lap_cdf((np.asarray(s, np.float64) - b) / alpha)))


def _excess_exact(s_dec, b, alpha_dec, k_dec):
    """M(b) - k in 60-digit decimal arithmetic, from the definition with the
    constant 1 of every above-b term grouped into an exact count, so a flat
    stretch of M (a gap of hundreds of alpha, where the exponentials are
    ~1e-400) still has the right sign."""
    half = Decimal(1) / 2
    cnt = 0
    below = Decimal(0)
    above = Decimal(0)
    for si in s_dec:
        x = (si - b) / alpha_dec
        if x <= 0:
            below += half * x.exp()
        else:
            cnt += 1
            above += half * (-x).exp()
    return (Decimal(cnt) - k_dec) + (below - above)


def bisect_threshold(s, k, alpha, iters=400):
    """Brute force: bisection on M(b) = k straight from the definition, in
    60-digit decimal arithmetic (no sort, no recurrences, no closed form)."""
    with localcontext() as ctx:
        ctx.prec = 60
        s_dec = [Decimal(float(v)) for v in np.asarray(s, np.float64)]
        a = Decimal(float(alpha))
        kk = Decimal(float(k))
        lo = min(s_dec) - a
        hi = max(s_dec) + a
        while _excess_exact(s_dec, lo, a, kk) < 0:
            lo -= (hi - lo) + a
        while _excess_exact(s_dec, hi, a, kk) > 0:
            hi += (hi - lo) + a
        stop = Decimal("1e-19") * (abs(lo) + abs(hi)) + Decimal("1e-19") * a
        for _ in range(iters):
            if hi - lo <= stop:
                break
            mid = (lo + hi) / 2
            if _excess_exact(s_dec, mid, a, kk) >= 0:
                lo = mid
            else:
                hi = mid
        return float((lo + hi) / 2)


def laplace_quantile(q):
    """Inverse of the standard Laplace CDF."""
    return math.log(2 * q) if q <= 0.5 else -math.log(2 * (1 - q))


# --------------------------------------------------------------------------
# the battery
# --------------------------------------------------------------------------
def pin_bisection(orc, cases=90, seed=1234):
    """Oracle b equals brute-force bisection on tiny inputs (n <= 64), incl. ties."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for c in range(cases):
        n = int(rng.integers(1, 65))
        alpha = float(10 ** rng.uniform(-3, 1))
        s = rng.normal(size=n) * float(10 ** rng.uniform(-2, 1))
        if c % 3 == 0:  # ties
            s = np.round(s * 2) / 2
        if c % 2 == 0 and n > 1:
            k = float(rng.integers(1, n))
        else:
            k = float(rng.uniform(0.01, n - 0.01)) if n > 1 else float(rng.uniform(0.01, 0.99))
        b = orc.threshold(s, k, alpha)
        bb = bisect_threshold(s, k, alpha)
        err = abs(b - bb) / alpha
        worst = max(worst, err)
        assert err <= 1e-9 * max(1.0, 1.0 / k) + 1e-12 * np.abs(s).max() / alpha, (c, n, k, alpha, b, bb)
    return worst


def pin_two_point_midpoint(orc):
    """n=2, k=1: by the symmetry F(-x) = 1 - F(x), b is the midpoint exactly."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        s = rng.normal(size=2) * 3
        alpha = float(10 ** rng.uniform(-4, 1))
        b = orc.threshold(s, 1.0, alpha)
        assert abs(b - s.mean()) <= 4e-16 * (1 + np.abs(s).max()), (s, alpha, b)


def pin_all_equal(orc):
    """All scores equal s0: p_i = k/n, b = s0 - alpha F^{-1}(k/n)."""
    for n, k, alpha, s0 in [(1, 0.3, 1.0, 0.0), (1, 0.9, 0.5, 2.0), (10, 3.0, 0.1, -1.5),
                            (10, 7.5, 2.0, 4.0), (64, 32.0, 0.01, 1.0), (1000, 1.0, 1e-3, 0.25)]:
        s = np.full(n, s0)
        p, b = orc.forward(s, k, alpha)
        expect = s0 - alpha * laplace_quantile(k / n)
        assert abs(b - expect) <= 1e-13 * (1 + abs(s0)), (n, k, b, expect)
        assert np.max(np.abs(p - k / n)) <= 1e-13


def pin_symmetric_sets(orc):
    """Scores symmetric about c with k = n/2 put b at c exactly; reflecting s
    and k -> n-k reflects b."""
    rng = np.random.default_rng(11)
    for _ in range(40):
        half = rng.normal(size=int(rng.integers(1, 30)))
        c = float(rng.normal())
        s = np.concatenate([c + half, c - half])
        alpha = float(10 ** rng.uniform(-3, 1))
        b = orc.threshold(s, s.size / 2, alpha)
        assert abs(b - c) <= 1e-12 * (1 + np.abs(s).max()), (b, c)
        t = rng.normal(size=int(rng.integers(2, 40)))
        k = float(rng.uniform(0.1, t.size - 0.1))
        b1 = orc.threshold(t, k, alpha)
        b2 = orc.threshold(-t, t.size - k, alpha)
        assert abs(b1 + b2) <= 1e-10 * alpha + 1e-13 * (1 + np.abs(t).max()), (b1, b2)


def pin_logsumexp_extremes(orc):
    """Root beyond every score has the library closed form:
    above all:  b = alpha*logsumexp(s/alpha) - alpha*ln(2k)
    below all:  b = -alpha*logsumexp(-s/alpha) + alpha*ln(2(n-k))."""
    rng = np.random.default_rng(5)
    for _ in range(40):
        n = int(rng.integers(1, 200))
        s = rng.normal(size=n)
        rngw = float(s.max() - s.min())
        alpha = float(10 ** rng.uniform(-2, 0.5))
        k = float(rng.uniform(1e-3, 0.9)) * 0.5 * math.exp(-rngw / alpha)
        k = max(k, 1e-300)
        b_hi = alpha * logsumexp(s / alpha) - alpha * math.log(2 * k)
        assert b_hi >= s.max()
        b = orc.threshold(s, k, alpha)
        assert abs(b - b_hi) <= 1e-12 * (abs(b_hi) + alpha * 50), (b, b_hi)
        # below every score: keep n - k2 = k representable next to n
        alpha2 = max(alpha, rngw / 5.0, 1e-3)
        kl = float(rng.uniform(1e-3, 0.9)) * 0.5 * math.exp(-rngw / alpha2)
        k2 = n - kl
        b_lo = -alpha2 * logsumexp(-s / alpha2) + alpha2 * math.log(2 * (n - k2))
        assert b_lo <= s.min()
        b2 = orc.threshold(s, k2, alpha2)
        assert abs(b2 - b_lo) <= 1e-12 * (abs(b_lo) + alpha2 * 50) + 1e-10 * alpha2 * n, (b2, b_lo)


def pin_zero_temperature(orc):
    """alpha -> 0: b tends to the midpoint of the k-th and (k+1)-th largest
    scores and p to the hard top-k indicator (section 2.3)."""
    rng = np.random.default_rng(3)
    for _ in range(30):
        n = int(rng.integers(2, 80))
        s = rng.permutation(np.arange(n, dtype=np.float64) * 0.37 + rng.uniform(0, 0.3, size=n))
        gap = np.min(np.diff(np.sort(s)))
        k = int(rng.integers(1, n))
        alpha = 1e-6 * gap
        p, b = orc.forward(s, float(k), alpha)
        xs = np.sort(s)[::-1]
        mid = 0.5 * (xs[k - 1] + xs[k])
        assert abs(b - mid) <= alpha * math.log(n) + 1e-14 * (1 + abs(mid)), (b, mid)
        hard = np.zeros(n)
        hard[np.argsort(-s)[:k]] = 1.0
        assert np.max(np.abs(p - hard)) <= 1e-6


def pin_large_temperature(orc):
    """alpha >> spread with k = n/2: F(x) = 1/2 + x/2 + O(x^2) near 0, so b
    approaches the mean of the scores."""
    rng = np.random.default_rng(9)
    for _ in range(20):
        s = rng.normal(size=int(rng.integers(2, 100)))
        spread = float(np.ptp(s)) + 1e-3
        alpha = 1e6 * spread
        b = orc.threshold(s, s.size / 2, alpha)
        assert abs(b - s.mean()) <= 10 * spread ** 2 / alpha + 1e-12 * alpha, (b, s.mean())


def pin_mass_and_order(orc):
    """sum p = k (definition evaluated independently); p monotone in s; equal
    scores get equal p."""
    rng = np.random.default_rng(21)
    for trial in range(12):
        n = int(rng.integers(2, 20000))
        s = rng.normal(size=n)
        if trial % 2:
            s = np.round(s, 2)
        alpha = float(10 ** rng.uniform(-3, 0.5))
        k = float(rng.uniform(0.5, n - 0.5))
        p, b = orc.forward(s, k, alpha)
        m = float(np.sum(lap_cdf((s - b) / alpha)))
        assert abs(m - k) <= 1e-9 * max(1.0, k), (m, k)
        assert abs(float(np.sum(p)) - k) <= 1e-9 * max(1.0, k)
        order = np.argsort(s, kind="stable")
        assert np.all(np.diff(p[order]) >= 0)
        _, inv = np.unique(s, return_inverse=True)
        for u in np.unique(inv)[:50]:
            vals = p[inv == u]
            assert np.all(vals == vals[0])


def pin_invariances(orc):
    """Shift, scale and permutation invariance of the definition."""
    rng = np.random.default_rng(31)
    for _ in range(20):
        n = int(rng.integers(2, 300))
        s = rng.normal(size=n)
        alpha = float(10 ** rng.uniform(-2, 0.5))
        k = float(rng.uniform(0.2, n - 0.2))
        p, b = orc.forward(s, k, alpha)
        c = float(rng.normal() * 4)
        p2, b2 = orc.forward(s + c, k, alpha)
        assert abs(b2 - (b + c)) <= 1e-12 * (1 + abs(b) + abs(c)) + 1e-10 * alpha
        assert np.max(np.abs(p2 - p)) <= 1e-9
        p3, b3 = orc.forward(2.0 * s, k, 2.0 * alpha)
        assert abs(b3 - 2.0 * b) <= 1e-12 * (1 + abs(b))
        assert np.max(np.abs(p3 - p)) <= 1e-12
        perm = rng.permutation(n)
        p4, b4 = orc.forward(s[perm], k, alpha)
        assert b4 == b or abs(b4 - b) <= 1e-13 * (1 + abs(b))
        assert np.max(np.abs(p4 - p[perm])) <= 1e-12


def pin_vjp(orc):
    """Backward equals central finite differences of the forward; the
    gradient sums to zero (shift invariance) and the Jacobian is symmetric."""
    rng = np.random.default_rng(41)
    for _ in range(10):
        n = int(rng.integers(2, 48))
        s = rng.normal(size=n)
        alpha = float(10 ** rng.uniform(-1, 0.5))
        k = float(rng.uniform(0.3, n - 0.3))
        u = rng.normal(size=n)
        v = rng.normal(size=n)
        _, b = orc.forward(s, k, alpha)
        gu = orc.backward(u, s, alpha, b)
        gv = orc.backward(v, s, alpha, b)
        h = 1e-6 * alpha
        fd = np.empty(n)
        for i in range(n):
            e = np.zeros(n)
            e[i] = h
            pp, _ = orc.forward(s + e, k, alpha)
            pm, _ = orc.forward(s - e, k, alpha)
            fd[i] = float(np.dot(u, pp - pm)) / (2 * h)
        rel = np.linalg.norm(gu - fd) / max(np.linalg.norm(fd), 1e-300)
        assert rel <= 1e-5, rel
        assert abs(float(np.sum(gu))) <= 1e-9 * (np.abs(gu).sum() + 1e-300)
        assert abs(float(np.dot(v, gu)) - float(np.dot(u, gv))) <= 1e-9 * (
            np.linalg.norm(u) * np.linalg.norm(gv) + 1e-300)


def pin_vjp_underflow(orc):
    """When alpha is so small that every d_i underflows, the VJP is 0 (not
    0/0); with partial underflow it still equals the definition's G/D form."""
    for s, k, alpha in [(np.array([0.0, 1.0]), 1.0, 1e-4), (np.array([0.0, 1.0, 3.0, 7.0]), 2.0, 1e-5)]:
        _, b = orc.forward(s, k, alpha)
        g = np.arange(1.0, s.size + 1.0)
        gr = orc.backward(g, s, alpha, b)
        assert np.all(np.isfinite(gr)) and np.all(gr == 0.0), gr
    rng = np.random.default_rng(17)
    s = rng.normal(size=40)
    g = rng.normal(size=40)
    alpha = 0.01
    _, b = orc.forward(s, 10.0, alpha)
    d = 0.5 * np.exp(-np.abs(s - b) / alpha)
    naive = (d / alpha) * (g - np.sum(g * d) / np.sum(d))
    gr = orc.backward(g, s, alpha, b)
    assert np.max(np.abs(gr - naive)) <= 1e-9 * np.max(np.abs(naive))


def pin_mass(orc):
    """The selected mass M(b) = sum_i F((s_i - b)/alpha) (section 2.1), checked
    against what fixes it without re-typing it: F(0) = 1/2 (every score at b
    selects half a unit), F(x) + F(-x) = 1 (reflection: M_s(b) + M_{-s}(-b) = n),
    the one-sided closed forms beyond every score (scipy's logsumexp), the
    brute-force bisection root (60-digit decimal arithmetic) where the mass is
    k, shift invariance, and strict decrease in b."""
    rng = np.random.default_rng(77)
    for n, s0, alpha in [(1, 0.0, 1.0), (7, -2.5, 0.1), (1000, 0.25, 1e-3)]:
        m = orc.mass(np.full(n, s0), s0, alpha)
        assert abs(m - n / 2) <= 1e-12 * n, (n, m)
    for _ in range(30):
        half = rng.normal(size=int(rng.integers(1, 40)))
        c = float(rng.normal())
        s = np.concatenate([c + half, c - half])
        alpha = float(10 ** rng.uniform(-3, 1))
        assert abs(orc.mass(s, c, alpha) - s.size / 2) <= 1e-12 * s.size
    for _ in range(30):
        n = int(rng.integers(1, 300))
        s = rng.normal(size=n) * float(10 ** rng.uniform(-1, 1))
        alpha = float(10 ** rng.uniform(-2, 0.5))
        b = float(rng.normal() * 2)
        m1, m2 = orc.mass(s, b, alpha), orc.mass(-s, -b, alpha)
        assert abs(m1 + m2 - n) <= 1e-12 * n, (m1, m2, n)
        c = float(rng.normal() * 8)
        assert abs(orc.mass(s + c, b + c, alpha) - m1) <= 1e-9 * max(1.0, m1)
        # beyond every score the mass is one exponential sum
        hi = float(s.max()) + float(rng.uniform(0, 3)) * alpha
        lo = float(s.min()) - float(rng.uniform(0, 3)) * alpha
        m_hi = 0.5 * math.exp(logsumexp((s - hi) / alpha))
        m_lo = n - 0.5 * math.exp(logsumexp((lo - s) / alpha))
        assert abs(orc.mass(s, hi, alpha) - m_hi) <= 1e-12 * max(1.0, m_hi) * n, (hi, m_hi)
        assert abs(orc.mass(s, lo, alpha) - m_lo) <= 1e-12 * n, (lo, m_lo)
        # strictly decreasing in b
        bs = np.sort(rng.normal(size=8) * 2)
        ms = [orc.mass(s, float(x), alpha) for x in bs]
        assert all(ms[i] >= ms[i + 1] for i in range(7)), ms
        assert ms[0] > ms[-1] or bs[0] == bs[-1]
    for c in range(25):
        n = int(rng.integers(1, 40))
        s = rng.normal(size=n)
        if c % 3 == 0:
            s = np.round(s * 2) / 2
        alpha = float(10 ** rng.uniform(-2, 0.5))
        k = float(rng.uniform(0.05, n - 0.05)) if n > 1 else 0.5
        b = bisect_threshold(s, k, alpha)
        m = orc.mass(s, b, alpha)
        assert abs(m - k) <= 1e-9 * max(1.0, k), (n, k, alpha, m)


def kth_largest_by_counting(s, j):
    """The j-th largest score, by counting alone (no sort): v is it when fewer
    than j scores exceed v and at least j are at or above it."""
    s = [float(v) for v in s]
    for v in s:
        above = sum(1 for w in s if w > v)
        at_or_above = sum(1 for w in s if w >= v)
        if above < j <= at_or_above:
            return v
    raise AssertionError("no j-th largest")


def pin_dftopk(orc):
    """DFTopK comparator (DFTopK page, abstract; Fast LapSum summary, section
    2.3): b is the midpoint of the k-th and (k+1)-th largest scores, found
    here by counting on tiny inputs (ties included); LapSum's threshold tends
    to it as alpha -> 0 and its p to the hard top-k indicator; reflecting
    the scores with k -> n - k reflects b; shift, scale and permutation act
    on b as on the scores; and p_i = F((s_i - b)/alpha) sums to the
    definition's mass at b."""
    rng = np.random.default_rng(99)
    for c in range(60):
        n = int(rng.integers(2, 65))
        s = rng.normal(size=n)
        if c % 3 == 0:
            s = np.round(s * 2) / 2
        k = int(rng.integers(1, n))
        b = orc.dftopk_threshold(s, k)
        want = 0.5 * (kth_largest_by_counting(s, k) + kth_largest_by_counting(s, k + 1))
        assert b == want, (n, k, b, want)
        b2 = orc.dftopk_threshold(-s, n - k)
        assert b2 == -b, (b, b2)
        cc = float(rng.normal() * 3)
        assert abs(orc.dftopk_threshold(s + cc, k) - (b + cc)) <= 1e-12 * (1 + abs(b) + abs(cc))
        assert orc.dftopk_threshold(2.0 * s, k) == 2.0 * b
        assert orc.dftopk_threshold(s[rng.permutation(n)], k) == b
        alpha = float(10 ** rng.uniform(-2, 0.5))
        p, bp = orc.dftopk_forward(s, k, alpha)
        assert bp == b
        assert abs(float(np.sum(p)) - mass_def(s, b, alpha)) <= 1e-12 * n
        assert np.max(np.abs(p - lap_cdf((s - b) / alpha))) <= 1e-15
    for _ in range(20):
        n = int(rng.integers(2, 80))
        s = rng.permutation(np.arange(n, dtype=np.float64) * 0.37 + rng.uniform(0, 0.3, size=n))
        gap = float(np.min(np.diff(np.sort(s))))
        k = int(rng.integers(1, n))
        alpha = 1e-6 * gap
        b_lap = orc.threshold(s, float(k), alpha)
        b_dft = orc.dftopk_threshold(s, k)
        assert abs(b_lap - b_dft) <= alpha * math.log(n) + 1e-14 * (1 + abs(b_dft)), (b_lap, b_dft)
        p, _ = orc.dftopk_forward(s, k, alpha)
        hard = np.zeros(n)
        hard[np.argsort(-s)[:k]] = 1.0
        assert np.max(np.abs(p - hard)) <= 1e-6


ALL_PINS = [
    pin_bisection,
    pin_two_point_midpoint,
    pin_all_equal,
    pin_symmetric_sets,
    pin_logsumexp_extremes,
    pin_zero_temperature,
    pin_large_temperature,
    pin_mass_and_order,
    pin_invariances,
    pin_vjp,
    pin_vjp_underflow,
    pin_mass,
    pin_dftopk,
]
