"""GPU: the allocation-free encoder entry point (dfc_encode_device_noalloc),
called through the C ABI, against dfc_encode_device with a caller
workspace: byte-identical containers on two calls in a row, the second
with a smaller input (the fixed device array keeps the first call's
contents), and sizes past the fixed workspace refused before any work."""
import ctypes

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def with_workspace(src, p):
    """dfc_encode_device with a caller workspace (the existing entry point)."""
    n = src.numel()
    cap = dfc.encode_bound(n, p)
    wb = ctypes.c_uint64()
    assert dfc.library().dfc_encode_device_workspace(n, ctypes.byref(wb)) == dfc.OK
    dst = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    work = torch.empty(max(256, wb.value), dtype=torch.uint8, device="cuda")
    written = ctypes.c_uint64()
    s = dfc.library().dfc_encode_device(ctypes.c_void_p(src.data_ptr()), n, ctypes.byref(p), None,
                                        ctypes.c_void_p(dst.data_ptr()), cap, ctypes.c_void_p(work.data_ptr()),
                                        wb.value, ctypes.byref(written), None)
    assert s == dfc.OK
    torch.cuda.synchronize()
    return dst[: written.value].cpu().numpy()


def no_alloc(src, p, dst):
    written = ctypes.c_uint64()
    s = dfc.library().dfc_encode_device_noalloc(ctypes.c_void_p(src.data_ptr()), src.numel(), ctypes.byref(p), None,
                                                ctypes.c_void_p(dst.data_ptr()), dst.numel(), ctypes.byref(written),
                                                None)
    torch.cuda.synchronize()
    return s, written.value


@pytest.mark.parametrize("layout", [dfc.LAYOUT_FLAT, dfc.LAYOUT_ANS, dfc.LAYOUT_PANEL])
def test_two_calls_match_the_workspace_entry_point(layout):
    shapes = ((4096, 4096), (1024, 512)) if layout != dfc.LAYOUT_ANS else ((4096, 2048), (512, 768))
    for j, shape in enumerate(shapes):   # the second call is the smaller one
        x = synth.gaussian_with_outliers(shape, 0.02, (120, layout, j))
        src = torch.from_numpy(x.reshape(-1).view(np.int16)).cuda()
        p = dfc.default_params(rows=shape[0], cols=shape[1], layout=layout,
                               panel_k=256 if layout == dfc.LAYOUT_PANEL else 0,
                               ans_steps=256 if layout == dfc.LAYOUT_ANS else 0)
        want = with_workspace(src, p)
        dst = torch.full((dfc.encode_bound(x.size, p),), 0xA5, dtype=torch.uint8, device="cuda")
        s, size = no_alloc(src, p, dst)
        assert s == dfc.OK and size == want.size, (shape, s)
        assert np.array_equal(dst[:size].cpu().numpy(), want), shape
        assert np.array_equal(dst[:size].cpu().numpy(), dfc.encode(x, layout=layout, shape=shape,
                                                                   panel_k=p.panel_k, ans_steps=p.ans_steps)), shape


def test_inputs_past_the_fixed_workspace_are_refused():
    lib = dfc.library()
    n = 715_783_681   # the first n whose workspace exceeds DFC_NOALLOC_WORKSPACE_BYTES
    wb = ctypes.c_uint64()
    assert lib.dfc_encode_device_workspace(n, ctypes.byref(wb)) == dfc.OK and wb.value > 16 << 20
    assert lib.dfc_encode_device_workspace(n - 1, ctypes.byref(wb)) == dfc.OK and wb.value <= 16 << 20
    src = torch.empty(16, dtype=torch.int16, device="cuda")   # never read: the size check comes first
    dst = torch.empty(256, dtype=torch.uint8, device="cuda")
    written = ctypes.c_uint64()
    p = dfc.default_params()
    s = lib.dfc_encode_device_noalloc(ctypes.c_void_p(src.data_ptr()), n, ctypes.byref(p), None,
                                      ctypes.c_void_p(dst.data_ptr()), dst.numel(), ctypes.byref(written), None)
    assert s == dfc.ESIZE
