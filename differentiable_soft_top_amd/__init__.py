"""MI355X-native LapSum soft top-k.

    p, b = soft_topk(scores, k, alpha)

``scores``: 1-D fp32 tensor on a ROCm device.  ``p[i] = F((scores[i]-b)/alpha)``
with F the standard Laplace CDF and b (fp64, one-element device tensor) the
threshold at which ``p.sum() == k``.  ``p`` is differentiable with respect to
``scores`` through the library's analytic vector-Jacobian product.

This module only marshals arguments: tensors supply device memory and the
current stream; every step of the computation runs in the HIP library
(``libsofttopk.so``, C ABI in include/soft_topk.h).  There is no CPU path.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import Params, SoftTopKError, Stats  # noqa: F401

__all__ = ["soft_topk", "forward", "backward", "rows_forward", "rows_backward", "threshold_curve", "dftopk_forward",
           "Params", "Stats", "SoftTopKError", "default_params"]


def default_params() -> Params:
    return _lib.default_params()


def _stream_handle(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_scores(s):
    import torch
    if not isinstance(s, torch.Tensor) or s.device.type != "cuda":
        raise TypeError("scores must be a tensor on a ROCm device")
    if s.dtype != torch.float32 or s.dim() != 1 or not s.is_contiguous():
        raise TypeError("scores must be a contiguous 1-D float32 tensor")


def forward(s, k: float, alpha: float, params: Params | None = None, out_p=None, want_stats: bool = False,
            want_workspace: bool = False):
    """Run soft_topk_forward_ex; returns (p, b[, stats dict][, workspace]).  The workspace, passed on to
    backward(), lets it reuse what the forward recorded about saturated scores."""
    import torch
    _check_scores(s)
    lib = _lib.load()
    n = s.numel()
    pp = ctypes.byref(params) if params is not None else None
    ws_bytes = lib.soft_topk_workspace_bytes(n, pp)
    if ws_bytes == 0:
        raise SoftTopKError(_lib.EINVAL, "invalid size or params (n=%d)" % n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=s.device)
    p = out_p if out_p is not None else torch.empty_like(s)
    b = torch.empty(1, dtype=torch.float64, device=s.device)
    stats = Stats()
    # a stats record makes the call wait for the certification pass: only on request
    rc = lib.soft_topk_forward_ex(ctypes.c_void_p(s.data_ptr()), n, float(k), float(alpha),
                                  ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                  ctypes.c_void_p(ws.data_ptr()), ws_bytes, _stream_handle(s),
                                  pp, ctypes.byref(stats) if want_stats else None)
    _lib.check(rc, "soft_topk_forward")
    out = (p, b)
    if want_stats:
        out += (stats.as_dict(),)
    if want_workspace:
        out += (ws,)
    return out


def backward(grad_p, s, alpha: float, b, out=None, fwd_workspace=None):
    """Run soft_topk_backward_ex: (d_i/alpha)(g_i - G/D).  fwd_workspace: the forward's workspace
    (from forward(..., want_workspace=True)), or None to read the scores throughout."""
    import torch
    _check_scores(s)
    if grad_p.dtype != torch.float32 or grad_p.shape != s.shape or not grad_p.is_contiguous():
        raise TypeError("grad_p must be a contiguous float32 tensor shaped like scores")
    if b.dtype != torch.float64 or b.numel() != 1 or b.device != s.device:
        raise TypeError("b must be the one-element float64 device tensor from forward")
    lib = _lib.load()
    n = s.numel()
    ws_bytes = lib.soft_topk_backward_workspace_bytes(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=s.device)
    g = out if out is not None else torch.empty_like(s)
    fw = None if fwd_workspace is None else ctypes.c_void_p(fwd_workspace.data_ptr())
    fw_bytes = 0 if fwd_workspace is None else fwd_workspace.numel() * fwd_workspace.element_size()
    rc = lib.soft_topk_backward_ex(ctypes.c_void_p(grad_p.data_ptr()), ctypes.c_void_p(s.data_ptr()), n,
                                   float(alpha), ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                                   fw, fw_bytes, ctypes.c_void_p(ws.data_ptr()), ws_bytes, _stream_handle(s))
    _lib.check(rc, "soft_topk_backward")
    return g


def _check_rows(s):
    import torch
    if not isinstance(s, torch.Tensor) or s.dtype != torch.float32 or s.dim() != 2 or not s.is_contiguous():
        raise TypeError("scores must be a contiguous 2-D float32 tensor (rows x n_row)")
    if s.device.type != "cuda":
        raise TypeError("scores must live on a ROCm device")


def threshold_curve(s, alpha: float):
    """soft_topk_threshold_curve: returns (sorted scores fp32, mass fp64), mass[j] being the k that the
    threshold b = sorted[j] selects (non-increasing)."""
    import torch
    _check_scores(s)
    lib = _lib.load()
    n = s.numel()
    ws_bytes = lib.soft_topk_workspace_bytes(n, None)
    if ws_bytes == 0:
        raise SoftTopKError(_lib.EINVAL, "invalid size (n=%d)" % n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=s.device)
    xs = torch.empty_like(s)
    mass = torch.empty(n, dtype=torch.float64, device=s.device)
    rc = lib.soft_topk_threshold_curve(ctypes.c_void_p(s.data_ptr()), n, float(alpha), ctypes.c_void_p(xs.data_ptr()),
                                       ctypes.c_void_p(mass.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                                       _stream_handle(s))
    _lib.check(rc, "soft_topk_threshold_curve")
    return xs, mass


def dftopk_forward(s, k: int, alpha: float, out_p=None):
    """DFTopK comparator (soft_topk_dftopk_forward): b at the midpoint of the k-th and (k+1)-th
    largest scores, p = F((s - b)/alpha).  Returns (p, b, mass) with mass = sum p (fp64, device);
    mass - k is the drift from the budget.  Not differentiable (no backward)."""
    import torch
    _check_scores(s)
    lib = _lib.load()
    n = s.numel()
    ws_bytes = lib.soft_topk_dftopk_workspace_bytes(n)
    if ws_bytes == 0:
        raise SoftTopKError(_lib.EINVAL, "invalid size (n=%d)" % n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=s.device)
    p = out_p if out_p is not None else torch.empty_like(s)
    b = torch.empty(1, dtype=torch.float64, device=s.device)
    m = torch.empty(1, dtype=torch.float64, device=s.device)
    rc = lib.soft_topk_dftopk_forward(ctypes.c_void_p(s.data_ptr()), n, float(k), float(alpha),
                                      ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                      ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                                      _stream_handle(s))
    _lib.check(rc, "soft_topk_dftopk_forward")
    return p, b, m


def rows_forward(s, k: float, alpha: float, out_p=None):
    """Batched rows (soft_topk_rows_forward): s is rows x n_row; returns (p, b) with b one fp64
    threshold per row.  A row holding a non-finite score gets b = NaN and p = NaN."""
    import torch
    _check_rows(s)
    lib = _lib.load()
    rows, n_row = s.shape
    ws_bytes = lib.soft_topk_rows_workspace_bytes(rows, n_row)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=s.device)
    p = out_p if out_p is not None else torch.empty_like(s)
    b = torch.empty(rows, dtype=torch.float64, device=s.device)
    rc = lib.soft_topk_rows_forward(ctypes.c_void_p(s.data_ptr()), rows, n_row, float(k), float(alpha),
                                    ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                    ctypes.c_void_p(ws.data_ptr()), ws_bytes, _stream_handle(s))
    _lib.check(rc, "soft_topk_rows_forward")
    return p, b


def rows_backward(grad_p, s, alpha: float, b, out=None):
    """Backward of rows_forward (soft_topk_rows_backward), each row with its own D and G."""
    import torch
    _check_rows(s)
    if grad_p.dtype != torch.float32 or grad_p.shape != s.shape or not grad_p.is_contiguous():
        raise TypeError("grad_p must be a contiguous float32 tensor shaped like scores")
    if b.dtype != torch.float64 or b.numel() != s.shape[0] or b.device != s.device:
        raise TypeError("b must be the per-row float64 device tensor from rows_forward")
    lib = _lib.load()
    rows, n_row = s.shape
    ws_bytes = lib.soft_topk_rows_workspace_bytes(rows, n_row)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=s.device)
    g = out if out is not None else torch.empty_like(s)
    rc = lib.soft_topk_rows_backward(ctypes.c_void_p(grad_p.data_ptr()), ctypes.c_void_p(s.data_ptr()), rows,
                                     n_row, float(alpha), ctypes.c_void_p(b.data_ptr()),
                                     ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                                     _stream_handle(s))
    _lib.check(rc, "soft_topk_rows_backward")
    return g


def _function():
    import torch

    class _SoftTopK(torch.autograd.Function):
        @staticmethod
        def forward(ctx, s, k, alpha, params):
            p, b, ws = forward(s, k, alpha, params, want_workspace=True)
            # keep only what the backward reads (status block and segment
            # record), not the sort and band buffers of the whole workspace
            rec = ws[:_lib.load().soft_topk_record_bytes(s.numel())].clone()
            del ws
            ctx.save_for_backward(s, b, rec)
            ctx.alpha = float(alpha)
            ctx.mark_non_differentiable(b)
            return p, b

        @staticmethod
        def backward(ctx, gp, gb):
            s, b, ws = ctx.saved_tensors
            if gp is None:
                return None, None, None, None
            return backward(gp.contiguous(), s, ctx.alpha, b, fwd_workspace=ws), None, None, None

    return _SoftTopK


_FN = None


def soft_topk(s, k: float, alpha: float, params: Params | None = None):
    """Differentiable LapSum soft top-k: returns (p, b)."""
    global _FN
    if _FN is None:
        _FN = _function()
    return _FN.apply(s, k, alpha, params)
