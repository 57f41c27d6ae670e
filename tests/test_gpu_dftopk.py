"""GPU parity of the DFTopK comparator (soft_topk_dftopk_forward) against the
fp64 oracle's DFTopK functions.

Bars: b is the midpoint of two fp32 order statistics computed in fp64 on both
sides, so it must agree bit for bit; p within 1e-5 element by element (the
emission is the LapSum operator's, fp64 arithmetic rounded to fp32); the
returned fp64 mass within 1e-9 * n of the oracle's mass at the same b.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import differentiable_soft_top_amd as stk  # noqa: E402
from differentiable_soft_top_amd import _lib  # noqa: E402
from differentiable_soft_top_amd.workloads import draw_scores, make_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    return torch.device("cuda:0")


def check(dev, s_np, k, alpha, tag):
    print("[dftopk] %s n=%d k=%d alpha=%g" % (tag, s_np.size, k, alpha), flush=True)
    s = torch.from_numpy(s_np).to(dev)
    p, b, m = stk.dftopk_forward(s, k, alpha)
    torch.cuda.synchronize()
    p_ref, b_ref = O.dftopk_forward(s_np, k, alpha)
    b_gpu = float(b.item())
    assert b_gpu == b_ref, (tag, b_gpu, b_ref)
    p_np = p.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(p_np - p_ref)) <= 1e-5, tag
    m_ref = O.mass(s_np, b_ref, alpha)
    assert abs(float(m.item()) - m_ref) <= 1e-9 * s_np.size, (tag, float(m.item()), m_ref)
    return b_gpu, float(m.item())


CASES = [
    ("c1", None, None),
    ("c2", 100_003, None),
    ("c3", 200_001, None),
    ("c4", 300_007, None),     # U(0,1) in fp32: many exact ties
    ("c5", 100_000, None),     # 60% tied at 0.5, k inside the tie
    ("c2", 1_000_000, None),
]


@pytest.mark.parametrize("name,n,_", CASES, ids=["%s-%s" % (a, b) for a, b, _ in CASES])
def test_dftopk_matches_oracle(dev, name, n, _):
    s_np, k, alpha, w = make_workload(name, n=n)
    check(dev, s_np, int(k), alpha, "%s-%s" % (name, n))


@pytest.mark.parametrize("n", [2, 3, 17, 64, 1000, 8191, 8192, 8193, 16385, 65537])
def test_dftopk_sizes_and_extreme_k(dev, n):
    s_np = draw_scores("normal", n, seed=n)
    for k in sorted({1, n // 2 if n > 2 else 1, n - 1}):
        check(dev, s_np, k, 0.1, "normal-%d-k%d" % (n, k))
    t = np.round(s_np * 4).astype(np.float32) / 4  # heavy ties
    check(dev, t, max(1, n // 3), 0.05, "ties-%d" % n)


def test_dftopk_structured(dev):
    n = 50_001
    base = draw_scores("normal", n, seed=3)
    check(dev, np.full(n, 0.25, np.float32), 100, 0.1, "equal")
    check(dev, np.sort(base), 777, 0.1, "sorted")
    check(dev, np.sort(base)[::-1].copy(), 777, 0.1, "reversed")
    check(dev, (base * 1e-30).astype(np.float32), 5000, 1e-31, "tiny")
    neg = -np.abs(base)
    neg[::7] = -0.0
    check(dev, neg.astype(np.float32), 20_000, 0.5, "signed-zeros")


def test_dftopk_nonfinite(dev):
    """A NaN anywhere makes b, every p and the mass NaN; infinities are
    ordered like other values (two +inf on top with k = 1: b = +inf)."""
    n = 40_000
    s_np = draw_scores("normal", n, seed=5)
    s_np[12_345] = np.nan
    s = torch.from_numpy(s_np).to(dev)
    p, b, m = stk.dftopk_forward(s, 10, 0.1)
    torch.cuda.synchronize()
    assert np.isnan(float(b.item())) and np.isnan(float(m.item()))
    assert np.all(np.isnan(p.cpu().numpy()))
    t_np = draw_scores("normal", n, seed=6)
    t_np[:2] = np.inf
    _, b2, _ = stk.dftopk_forward(torch.from_numpy(t_np).to(dev), 1, 0.1)
    torch.cuda.synchronize()
    assert float(b2.item()) == float("inf")


def test_dftopk_rejects_bad_arguments(dev):
    lib = _lib.load()
    s = torch.zeros(100, device=dev)
    p = torch.empty_like(s)
    b = torch.empty(1, dtype=torch.float64, device=dev)
    ws = torch.empty(lib.soft_topk_dftopk_workspace_bytes(100), dtype=torch.uint8, device=dev)
    v = ctypes.c_void_p
    for k, alpha in [(0.0, 0.1), (100.0, 0.1), (2.5, 0.1), (5.0, 0.0), (5.0, float("nan"))]:
        rc = lib.soft_topk_dftopk_forward(v(s.data_ptr()), 100, k, alpha, v(p.data_ptr()), v(b.data_ptr()), None,
                                          v(ws.data_ptr()), ws.numel(), None)
        assert rc == _lib.EINVAL, (k, alpha)
    rc = lib.soft_topk_dftopk_forward(v(s.data_ptr()), 100, 5.0, 0.1, v(p.data_ptr()), v(b.data_ptr()), None,
                                      v(ws.data_ptr()), 16, None)
    assert rc == _lib.EWORKSPACE
    assert lib.soft_topk_dftopk_workspace_bytes(1) == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_dftopk_full_size(dev, name):
    """The benchmark workloads at full size, every element; the mass drift
    (mass - k) is printed for the record."""
    s_np, k, alpha, w = make_workload(name)
    b, m = check(dev, s_np, int(k), alpha, name)
    print("[dftopk] %s b=%.12g mass=%.6f k=%d drift=%.4g (%.4g of k)" % (name, b, m, k, m - k, (m - k) / k),
          flush=True)
