"""ctypes loader for ``libsofttopk.so`` (the C ABI of include/soft_topk.h).

Argument marshalling only.  If the library is not built, loading raises: there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsofttopk.so")

OK, EINVAL, ENONFINITE, EWORKSPACE, EHIP, ESOLVE = 0, 1, 2, 3, 4, 5
PATH_BRACKET, PATH_WIDENED, PATH_FULLSORT, PATH_SINGLE, PATH_ALL_SCORES = 1, 2, 3, 4, 5
BAND_DIRECT, BAND_BUCKETS, BAND_REFINE, BAND_REFINE_STEPS = 1, 2, 3, 4
REJECT_LOW, REJECT_HIGH, REJECT_OVERFLOW, REJECT_BUCKET, REJECT_MASS = 1, 2, 4, 8, 16


class Params(ctypes.Structure):
    _fields_ = [
        ("seed", ctypes.c_uint64),
        ("samples", ctypes.c_int32),
        ("z", ctypes.c_double),
        ("band_capacity", ctypes.c_int64),
        ("max_widen", ctypes.c_int32),
        ("force_path", ctypes.c_int32),
        ("mass_tolerance", ctypes.c_double),
        ("verify_mass", ctypes.c_int32),
        ("band_route", ctypes.c_int32),
    ]


class Stats(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("rounds", ctypes.c_int32),
        ("reject_mask", ctypes.c_int32),
        ("band_route", ctypes.c_int32),
        ("a_left", ctypes.c_float),
        ("a_right", ctypes.c_float),
        ("n_left", ctypes.c_int64),
        ("n_band", ctypes.c_int64),
        ("n_right", ctypes.c_int64),
        ("mass_at_left", ctypes.c_double),
        ("mass_at_right", ctypes.c_double),
        ("b", ctypes.c_double),
        ("mass", ctypes.c_double),
        ("refine_passes", ctypes.c_int32),
        ("pad", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class SoftTopKError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lib = None


def load():
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libsofttopk.so is not built (expected at %s); run `python -c "
            "'import __graft_entry__ as g; g.build()'` from the repository root" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, dp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i64, i32, dbl, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
    lib.soft_topk_default_params.argtypes = [ctypes.POINTER(Params)]
    lib.soft_topk_default_params.restype = None
    lib.soft_topk_workspace_bytes.argtypes = [i64, ctypes.POINTER(Params)]
    lib.soft_topk_workspace_bytes.restype = sz
    lib.soft_topk_record_bytes.argtypes = [i64]
    lib.soft_topk_record_bytes.restype = sz
    lib.soft_topk_backward_workspace_bytes.argtypes = [i64]
    lib.soft_topk_backward_workspace_bytes.restype = sz
    lib.soft_topk_forward.argtypes = [fp, i64, dbl, dbl, fp, dp, vp, sz, vp]
    lib.soft_topk_forward.restype = ctypes.c_int
    lib.soft_topk_forward_ex.argtypes = [fp, i64, dbl, dbl, fp, dp, vp, sz, vp,
                                         ctypes.POINTER(Params), ctypes.POINTER(Stats)]
    lib.soft_topk_forward_ex.restype = ctypes.c_int
    lib.soft_topk_backward.argtypes = [fp, fp, i64, dbl, dp, fp, vp, sz, vp]
    lib.soft_topk_backward.restype = ctypes.c_int
    lib.soft_topk_backward_ex.argtypes = [fp, fp, i64, dbl, dp, fp, vp, sz, vp, sz, vp]
    lib.soft_topk_backward_ex.restype = ctypes.c_int
    lib.soft_topk_backward_noalloc.argtypes = [fp, fp, i64, dbl, dp, fp, vp]
    lib.soft_topk_backward_noalloc.restype = ctypes.c_int
    lib.soft_topk_dftopk_forward.argtypes = [fp, i64, dbl, dbl, fp, dp, dp, vp, sz, vp]
    lib.soft_topk_dftopk_forward.restype = ctypes.c_int
    lib.soft_topk_dftopk_workspace_bytes.argtypes = [i64]
    lib.soft_topk_dftopk_workspace_bytes.restype = sz
    lib.soft_topk_rows_forward.argtypes = [fp, i64, i64, dbl, dbl, fp, dp, vp, sz, vp]
    lib.soft_topk_rows_forward.restype = ctypes.c_int
    lib.soft_topk_rows_backward.argtypes = [fp, fp, i64, i64, dbl, dp, fp, vp, sz, vp]
    lib.soft_topk_rows_backward.restype = ctypes.c_int
    lib.soft_topk_threshold_curve.argtypes = [fp, i64, dbl, fp, dp, vp, sz, vp]
    lib.soft_topk_threshold_curve.restype = ctypes.c_int
    lib.soft_topk_rows_workspace_bytes.argtypes = [i64, i64]
    lib.soft_topk_rows_workspace_bytes.restype = sz
    lib.soft_topk_strerror.argtypes = [ctypes.c_int]
    lib.soft_topk_strerror.restype = ctypes.c_char_p
    lib.soft_topk_last_hip_error.argtypes = []
    lib.soft_topk_last_hip_error.restype = ctypes.c_int
    lib.soft_topk_bracket_ranks.argtypes = [i64, dbl, dbl, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.soft_topk_bracket_ranks.restype = ctypes.c_int
    lib.soft_topk_debug_sample.argtypes = [fp, i64, dbl, ctypes.c_uint64, i32, fp, vp]
    lib.soft_topk_debug_sample.restype = ctypes.c_int
    lib.soft_topk_profile_kernel_count.argtypes = []
    lib.soft_topk_profile_kernel_count.restype = ctypes.c_int
    lib.soft_topk_profile_kernel_name.argtypes = [ctypes.c_int]
    lib.soft_topk_profile_kernel_name.restype = ctypes.c_char_p
    lib.soft_topk_profile_begin.argtypes = [ctypes.c_uint32]
    lib.soft_topk_profile_begin.restype = ctypes.c_int
    lib.soft_topk_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.soft_topk_profile_end.restype = ctypes.c_int
    _lib = lib
    return lib


def kernel_names():
    lib = load()
    return [lib.soft_topk_profile_kernel_name(i).decode() for i in range(lib.soft_topk_profile_kernel_count())]


def profile_begin(names):
    """Start timing the named kernels (event pairs around each launch)."""
    all_names = kernel_names()
    mask = 0
    for nm in names:
        mask |= 1 << all_names.index(nm)
    check(load().soft_topk_profile_begin(mask), "soft_topk_profile_begin")


def profile_end():
    """Stop timing; return {kernel: (total_ms, launches)} for timed kernels."""
    lib = load()
    cnt = lib.soft_topk_profile_kernel_count()
    ms = (ctypes.c_double * cnt)()
    nl = (ctypes.c_int64 * cnt)()
    check(lib.soft_topk_profile_end(ms, nl), "soft_topk_profile_end")
    names = kernel_names()
    return {names[i]: (ms[i], nl[i]) for i in range(cnt) if nl[i] > 0}


def check(rc: int, what: str):
    if rc != OK:
        lib = load()
        msg = "%s failed: %s (code %d)" % (what, lib.soft_topk_strerror(rc).decode(), rc)
        if rc == EHIP:
            msg += ", hip error %d" % lib.soft_topk_last_hip_error()
        raise SoftTopKError(rc, msg)


def default_params() -> Params:
    p = Params()
    load().soft_topk_default_params(ctypes.byref(p))
    return p


def bracket_ranks(m: int, q: float, z: float):
    lib = load()
    rl, rr = ctypes.c_int64(0), ctypes.c_int64(0)
    check(lib.soft_topk_bracket_ranks(int(m), float(q), float(z), ctypes.byref(rl), ctypes.byref(rr)),
          "soft_topk_bracket_ranks")
    return rl.value, rr.value
