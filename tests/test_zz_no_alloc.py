"""The allocation-free backward (soft_topk_backward_noalloc) through the C ABI
against soft_topk_backward, the entry point whose kernels it runs with its
scratch in a fixed per-GPU array instead of a workspace: two calls in a row,
the second with a smaller input (the array keeps the first call's partials),
then a short vector (the one-work-group route).  Same kernels and grid, so
the outputs must agree bit for bit; each is also held to the oracle's
gradient (rel-L2 <= 1e-4)."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from differentiable_soft_top_amd import _lib  # noqa: E402
from differentiable_soft_top_amd.workloads import draw_grad, make_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    return torch.device("cuda:0")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def test_noalloc_backward_matches_workspace_backward(dev):
    lib = _lib.load()
    # n: the large-batch streaming shape (2^24 + ragged), then a smaller one, then one work-group
    for name, n in [("c4", (1 << 24) + 4099), ("c2", 100_003), ("c3", 5_000)]:
        print("[noalloc] %s n=%d" % (name, n), flush=True)
        s_np, k, alpha, w = make_workload(name, n=n)
        g_np = draw_grad(n, w.seed)
        b_ref = O.threshold(s_np, k, alpha)
        s = torch.from_numpy(s_np).to(dev)
        g = torch.from_numpy(g_np).to(dev)
        b = torch.tensor([b_ref], dtype=torch.float64, device=dev)
        out_ws = torch.full_like(s, float("nan"))
        out_na = torch.full_like(s, float("nan"))
        ws_bytes = lib.soft_topk_backward_workspace_bytes(n)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        _lib.check(lib.soft_topk_backward(_ptr(g), _ptr(s), n, alpha, _ptr(b), _ptr(out_ws), _ptr(ws), ws_bytes,
                                          _stream(dev)), "soft_topk_backward")
        _lib.check(lib.soft_topk_backward_noalloc(_ptr(g), _ptr(s), n, alpha, _ptr(b), _ptr(out_na), _stream(dev)),
                   "soft_topk_backward_noalloc")
        torch.cuda.synchronize()
        a_ws = out_ws.cpu().numpy()
        a_na = out_na.cpu().numpy()
        assert np.array_equal(a_ws.view(np.uint32), a_na.view(np.uint32)), name
        ref = O.backward(g_np, s_np, alpha, b_ref)
        rel = np.linalg.norm(a_na.astype(np.float64) - ref) / np.linalg.norm(ref)
        assert rel <= 1e-4, (name, rel)


def test_noalloc_backward_rejects_bad_arguments(dev):
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    assert lib.soft_topk_backward_noalloc(fake, fake, 0, 0.1, fake, fake, None) == _lib.EINVAL
    assert lib.soft_topk_backward_noalloc(fake, fake, 100, 0.0, fake, fake, None) == _lib.EINVAL
    assert lib.soft_topk_backward_noalloc(None, fake, 100, 0.1, fake, fake, None) == _lib.EINVAL
