"""Python access to the fp64 CPU oracle (``softtopk_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here imports, loads or calls
the GPU library, and the GPU library never calls this module.

The oracle computes the LapSum soft top-k operator exactly as defined in the
gist.science technical summary of "Fast LapSum: Exact Differentiable Top-k at
Million Scale" (section 2.1, the LapSum operator; section 2.2, the full-sort
solver).  All arithmetic is fp64; fp32 scores are widened exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "softtopk_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, ENONFINITE, ENOMEM = 0, 1, 2, 5


def build_oracle(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source with gcc into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    dbl = ctypes.c_double
    lib.oracle_mass.argtypes = [dp, i64, dbl, dbl]
    lib.oracle_mass.restype = dbl
    lib.oracle_threshold.argtypes = [dp, i64, dbl, dbl, dp]
    lib.oracle_threshold.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [dp, i64, dbl, dbl, dp, dp]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [dp, dp, i64, dbl, dbl, dp]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_dftopk_threshold.argtypes = [dp, i64, dbl, dp]
    lib.oracle_dftopk_threshold.restype = ctypes.c_int
    lib.oracle_dftopk_forward.argtypes = [dp, i64, dbl, dbl, dp, dp]
    lib.oracle_dftopk_forward.restype = ctypes.c_int
    return lib


def _as_f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).ravel())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__("oracle error code %d" % code)
        self.code = code


class Oracle:
    """The oracle's entry points bound to one compiled copy of the C source."""

    def __init__(self, lib_path: str):
        self.lib = _bind(ctypes.CDLL(lib_path))

    def threshold(self, s, k: float, alpha: float) -> float:
        """Exact threshold b with sum_i F((s_i - b)/alpha) = k (full-sort solver)."""
        x = _as_f64(s)
        b = ctypes.c_double(0.0)
        rc = self.lib.oracle_threshold(_ptr(x), x.size, float(k), float(alpha), ctypes.byref(b))
        if rc != OK:
            raise OracleError(rc)
        return b.value

    def forward(self, s, k: float, alpha: float):
        """Return (p, b): p_i = F((s_i - b)/alpha) in fp64, b in fp64."""
        x = _as_f64(s)
        p = np.empty_like(x)
        b = ctypes.c_double(0.0)
        rc = self.lib.oracle_forward(_ptr(x), x.size, float(k), float(alpha), _ptr(p), ctypes.byref(b))
        if rc != OK:
            raise OracleError(rc)
        return p, b.value

    def backward(self, g, s, alpha: float, b: float) -> np.ndarray:
        """Implicit-function VJP at threshold b: grad_l = (d_l/alpha)(g_l - G/D)."""
        x = _as_f64(s)
        gg = _as_f64(g)
        if gg.size != x.size:
            raise ValueError("g and s differ in length")
        out = np.empty_like(x)
        rc = self.lib.oracle_backward(_ptr(gg), _ptr(x), x.size, float(alpha), float(b), _ptr(out))
        if rc != OK:
            raise OracleError(rc)
        return out

    def mass(self, s, b: float, alpha: float) -> float:
        """Selected mass M(b) = sum_i F((s_i - b)/alpha), evaluated in fp64."""
        x = _as_f64(s)
        return self.lib.oracle_mass(_ptr(x), x.size, float(b), float(alpha))

    def dftopk_threshold(self, s, k: float) -> float:
        """DFTopK comparator: midpoint of the k-th and (k+1)-th largest scores."""
        x = _as_f64(s)
        b = ctypes.c_double(0.0)
        rc = self.lib.oracle_dftopk_threshold(_ptr(x), x.size, float(k), ctypes.byref(b))
        if rc != OK:
            raise OracleError(rc)
        return b.value

    def dftopk_forward(self, s, k: float, alpha: float):
        """DFTopK comparator: (p, b) with b the midpoint threshold, p_i = F((s_i - b)/alpha)."""
        x = _as_f64(s)
        p = np.empty_like(x)
        b = ctypes.c_double(0.0)
        rc = self.lib.oracle_dftopk_forward(_ptr(x), x.size, float(k), float(alpha), _ptr(p), ctypes.byref(b))
        if rc != OK:
            raise OracleError(rc)
        return p, b.value


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build_oracle()
        _default = Oracle(_LIB_PATH)
    return _default


def threshold(s, k: float, alpha: float) -> float:
    return default().threshold(s, k, alpha)


def forward(s, k: float, alpha: float):
    return default().forward(s, k, alpha)


def backward(g, s, alpha: float, b: float) -> np.ndarray:
    return default().backward(g, s, alpha, b)


def mass(s, b: float, alpha: float) -> float:
    return default().mass(s, b, alpha)


def dftopk_threshold(s, k: float) -> float:
    return default().dftopk_threshold(s, k)


def dftopk_forward(s, k: float, alpha: float):
    return default().dftopk_forward(s, k, alpha)
