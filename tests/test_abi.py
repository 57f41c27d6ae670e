"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol include/soft_topk.h declares, validates arguments before any
launch, sizes workspaces, and computes the bracket ranks from the binomial
law (checked against scipy's binomial distribution)."""
import ctypes
import os
import re

import pytest
from scipy.stats import binom, norm

from differentiable_soft_top_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "soft_topk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(soft_topk_[a-z_]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("soft_topk_forward", "soft_topk_backward", "soft_topk_workspace_bytes",
                 "soft_topk_backward_workspace_bytes", "soft_topk_forward_ex", "soft_topk_strerror"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror(lib):
    for code in range(0, 7):
        assert lib.soft_topk_strerror(code)


def test_forward_rejects_bad_arguments_before_launch(lib):
    # none of these touch the device: validation happens first
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x100000)
    good = dict(n=100, k=5.0, alpha=0.1)

    def call(s=fake, n=good["n"], k=good["k"], alpha=good["alpha"], p=fake, b=fake, w=ws, wb=1 << 40):
        return lib.soft_topk_forward(s, n, k, alpha, p, b, w, wb, None)

    assert call(n=0) == _lib.EINVAL
    assert call(n=-5) == _lib.EINVAL
    assert call(n=1 << 31) == _lib.EINVAL
    assert call(k=0.0) == _lib.EINVAL
    assert call(k=100.0) == _lib.EINVAL
    assert call(k=-1.0) == _lib.EINVAL
    assert call(k=float("nan")) == _lib.EINVAL
    assert call(alpha=0.0) == _lib.EINVAL
    assert call(alpha=-1.0) == _lib.EINVAL
    assert call(alpha=float("inf")) == _lib.EINVAL
    assert call(alpha=float("nan")) == _lib.EINVAL
    assert call(s=None) == _lib.EINVAL
    assert call(p=None) == _lib.EINVAL
    assert call(b=None) == _lib.EINVAL
    assert call(w=None) == _lib.EWORKSPACE
    assert call(wb=16) == _lib.EWORKSPACE
    assert call(w=ctypes.c_void_p(0x100010)) == _lib.EWORKSPACE  # not 256-byte aligned


def test_backward_rejects_bad_arguments_before_launch(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.soft_topk_backward(fake, fake, 0, 0.1, fake, fake, fake, 1 << 30, None) == _lib.EINVAL
    assert lib.soft_topk_backward(fake, fake, 10, 0.0, fake, fake, fake, 1 << 30, None) == _lib.EINVAL
    assert lib.soft_topk_backward(None, fake, 10, 0.1, fake, fake, fake, 1 << 30, None) == _lib.EINVAL
    assert lib.soft_topk_backward(fake, fake, 10, 0.1, None, fake, fake, 1 << 30, None) == _lib.EINVAL
    assert lib.soft_topk_backward(fake, fake, 10, 0.1, fake, fake, None, 1 << 30, None) == _lib.EWORKSPACE
    assert lib.soft_topk_backward(fake, fake, 10, 0.1, fake, fake, fake, 1, None) == _lib.EWORKSPACE


def test_threshold_curve_rejects_bad_arguments_before_launch(lib):
    fake = ctypes.c_void_p(0x1000)

    def curve(s=fake, n=100, alpha=0.1, xs=fake, m=fake, w=None, wb=0):
        return lib.soft_topk_threshold_curve(s, n, alpha, xs, m, w, wb, None)

    assert curve(n=0) == _lib.EINVAL
    assert curve(n=-5) == _lib.EINVAL
    assert curve(alpha=0.0) == _lib.EINVAL
    assert curve(alpha=float("inf")) == _lib.EINVAL
    assert curve(s=None) == _lib.EINVAL
    assert curve(xs=None) == _lib.EINVAL
    assert curve(m=None) == _lib.EINVAL
    # the forward's workspace size, 256-byte aligned
    assert curve() == _lib.EWORKSPACE
    need = lib.soft_topk_workspace_bytes(100, None)
    assert curve(w=ctypes.c_void_p(0x1001), wb=need) == _lib.EWORKSPACE
    assert curve(w=fake, wb=need - 1) == _lib.EWORKSPACE


def test_force_path_values(lib):
    p = _lib.Params()
    lib.soft_topk_default_params(ctypes.byref(p))
    fake = ctypes.c_void_p(0x1000)
    for v, ok in [(0, True), (_lib.PATH_BRACKET, True), (_lib.PATH_FULLSORT, True), (_lib.PATH_WIDENED, False),
                  (_lib.PATH_SINGLE, False), (7, False)]:
        p.force_path = v
        # a valid params block gets as far as the workspace check (none given)
        rc = lib.soft_topk_forward_ex(fake, 100, 5.0, 0.1, fake, fake, None, 0, None, ctypes.byref(p), None)
        assert rc == (_lib.EWORKSPACE if ok else _lib.EINVAL), (v, rc)


def test_rows_reject_bad_arguments_before_launch(lib):
    fake = ctypes.c_void_p(0x1000)

    def fwd(s=fake, rows=4, n_row=100, k=5.0, alpha=0.1, p=fake, b=fake, w=None, wb=0):
        return lib.soft_topk_rows_forward(s, rows, n_row, k, alpha, p, b, w, wb, None)

    assert fwd(rows=0) == _lib.EINVAL
    assert fwd(rows=-1) == _lib.EINVAL
    assert fwd(n_row=0) == _lib.EINVAL
    assert fwd(k=0.0) == _lib.EINVAL
    assert fwd(k=100.0) == _lib.EINVAL  # k must stay below n_row
    assert fwd(alpha=0.0) == _lib.EINVAL
    assert fwd(alpha=float("nan")) == _lib.EINVAL
    assert fwd(s=None) == _lib.EINVAL
    assert fwd(p=None) == _lib.EINVAL
    assert fwd(b=None) == _lib.EINVAL
    assert fwd(rows=1 << 31) == _lib.EINVAL  # one work-group per row

    def bwd(g=fake, s=fake, rows=4, n_row=100, alpha=0.1, b=fake, out=fake, w=None, wb=0):
        return lib.soft_topk_rows_backward(g, s, rows, n_row, alpha, b, out, w, wb, None)

    assert bwd(rows=0) == _lib.EINVAL
    assert bwd(alpha=-1.0) == _lib.EINVAL
    assert bwd(g=None) == _lib.EINVAL
    assert bwd(b=None) == _lib.EINVAL
    assert bwd(out=None) == _lib.EINVAL


def test_rows_workspace_sizes(lib):
    # every row length runs in the batched kernels: no workspace
    for n_row in (1, 64, 100, 4096, 8192, 8193, 10 ** 6):
        assert lib.soft_topk_rows_workspace_bytes(1000, n_row) == 0
    assert lib.soft_topk_rows_workspace_bytes(0, 100) == 0


def test_params_validation(lib):
    p = _lib.default_params()
    assert p.samples == 65536 and p.z == 5.0 and p.max_widen == 2 and p.force_path == 0
    assert lib.soft_topk_workspace_bytes(1000, ctypes.byref(p)) > 0
    for field, bad in [("samples", 10), ("samples", 1 << 20), ("z", 0.0), ("z", float("nan")),
                       ("max_widen", -1), ("force_path", 7), ("band_capacity", -3), ("verify_mass", 2),
                       ("band_route", 5)]:
        q = _lib.default_params()
        setattr(q, field, bad)
        assert lib.soft_topk_workspace_bytes(1000, ctypes.byref(q)) == 0, field


def test_workspace_sizes(lib):
    prev = 0
    for n in [1, 2, 3, 4, 5, 1000, 4096, 10 ** 6, 10 ** 7, 10 ** 8]:
        w = lib.soft_topk_workspace_bytes(n, None)
        assert w >= prev
        assert w >= 8 * n  # the full-sort route's two key arrays
        assert w % 256 == 0
        prev = w
        assert lib.soft_topk_backward_workspace_bytes(n) >= 16
    assert lib.soft_topk_workspace_bytes(0, None) == 0
    assert lib.soft_topk_workspace_bytes((1 << 31), None) == 0


@pytest.mark.parametrize("m,q,z", [(65536, 0.99, 5.0), (65536, 0.5, 5.0), (65536, 0.984375, 5.0),
                                   (4096, 0.9, 3.0), (65536, 1 - 1e-6, 5.0), (65536, 1e-6, 5.0),
                                   (1024, 0.999, 6.0), (262144, 0.99999, 5.0), (65536, 0.99, 10.0)])
def test_bracket_ranks_follow_the_binomial_law(m, q, z):
    """r_left is the largest rank with P(X <= r_left - 1) <= Phi(-z) and
    r_right the smallest with P(X >= r_right) <= Phi(-z), X ~ Binomial(m, q)
    (0 and m+1 stand for an open end)."""
    rl, rr = _lib.bracket_ranks(m, q, z)
    delta = norm.sf(z)
    X = binom(m, q)
    assert 0 <= rl < rr <= m + 1
    if rl >= 1:
        assert X.cdf(rl - 1) <= delta * (1 + 1e-6)
    if rl + 1 <= m:
        assert X.cdf(rl) > delta * (1 - 1e-6)
    if rr <= m:
        assert X.sf(rr - 1) <= delta * (1 + 1e-6)  # P(X >= rr)
    if rr - 1 >= 1:
        assert X.sf(rr - 2) > delta * (1 - 1e-6)  # P(X >= rr - 1)


def test_bracket_ranks_reject_bad_input():
    lib = _lib.load()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.soft_topk_bracket_ranks(0, 0.5, 5.0, ctypes.byref(a), ctypes.byref(b)) == _lib.EINVAL
    assert lib.soft_topk_bracket_ranks(100, 1.0, 5.0, ctypes.byref(a), ctypes.byref(b)) == _lib.EINVAL
    assert lib.soft_topk_bracket_ranks(100, 0.5, -1.0, ctypes.byref(a), ctypes.byref(b)) == _lib.EINVAL
