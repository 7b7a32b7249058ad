"""Direct C-ABI calls shared by the GPU tests: the _ex entry points with an explicit
leading dimension and an optional rfp4_force (None = the library's own choices), plus
the `force` fixture's patching of the binding."""

import ctypes
import functools

import gemm_rfp4_block_amd as R


def gemv_raw(wd, layout, n, k, xd, batch, ldx, y, ldy, force=None, stream=None):
    """rfp4_gemv_multi_ex with one part; returns the status."""
    wa = (ctypes.c_void_p * 1)(wd.data_ptr())
    na = (ctypes.c_int64 * 1)(n)
    ya = (ctypes.c_void_p * 1)(y.data_ptr())
    la = (ctypes.c_int64 * 1)(ldy)
    return R.lib().rfp4_gemv_multi_ex(1, wa, na, layout, k, R._ptr(xd), R._xdtype(xd), batch, ldx, ya, la,
                                      ctypes.byref(force) if force is not None else None, R._stream(stream))


def gemm_raw(wd, layout, n, k, ad, m, lda, c, ldc, force=None, stream=None):
    """rfp4_gemm_ex; returns the status."""
    return R.lib().rfp4_gemm_ex(R._ptr(wd), layout, n, k, R._ptr(ad), m, lda, R._ptr(c), ldc,
                                ctypes.byref(force) if force is not None else None, R._stream(stream))


def patch_binding(monkeypatch, force):
    """Route rfp4_gemv, rfp4_gemv_multi and rfp4_gemm of the binding through the _ex
    entry points with `force` for the rest of the test."""
    for name in ("rfp4_gemv", "rfp4_gemv_multi", "rfp4_gemm"):
        monkeypatch.setattr(R, name, functools.partial(getattr(R, name), force=force))
