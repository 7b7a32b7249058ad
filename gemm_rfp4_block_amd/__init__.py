"""Python binding of librfp4.so (ROCmFP4 decode, GEMV and GEMM on MI355X).

Argument marshalling only: each function passes tensor data pointers, sizes and the
current HIP stream to the C entry point of the same name (include/rfp4.h) and raises
on a non-zero status. Every step of the computation runs in the HIP kernels; there
is no CPU fallback. If librfp4.so has not been built, the first call raises.
"""

from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "librfp4.so")

RFP4_DUAL = 0
RFP4_FAST = 1
RFP4_F16 = 0
RFP4_BF16 = 1
RFP4_F32 = 2

RFP4_OK = 0
RFP4_ERR_NULL = 1
RFP4_ERR_SHAPE = 2
RFP4_ERR_UNSUPPORTED = 3
RFP4_ERR_NONFINITE_SCALE = 4
RFP4_ERR_HIP = 5
RFP4_ERR_SCRATCH = 6
GEMM_SCRATCH_BYTES = 32 << 20

EXPORTED = ("rfp4_block_bytes", "rfp4_row_bytes", "rfp4_status_string", "rfp4_validate",
            "rfp4_dequant", "rfp4_dequant_bf16", "rfp4_gemv", "rfp4_gemv_multi", "rfp4_gemm",
            "rfp4_gemm_dequant", "rfp4_quantize", "rfp4_gemv_multi_ex", "rfp4_gemm_ex",
            "rfp4_gemm_noalloc")
MAX_GEMV_PARTS = 8

# rfp4_gemv_kernel and rfp4_gemm_plan (include/rfp4.h)
GEMV_KERNEL = {"auto": 0, "dot": 1, "tiles": 2, "tall": 3, "no_tall": 4}
GEMM_PLAN = {"auto": 0, "main": 1, "msplit2": 2, "msplit3": 3, "msplit4": 4, "tail": 5, "tail2": 6,
             "tail4": 7, "nosplit": 8}


class Force(ctypes.Structure):
    """struct rfp4_force: kernel and plan overrides of the _ex entry points (all zero =
    the library's own choices)."""

    _fields_ = [("gemv_kernel", ctypes.c_int32), ("gemv_unit_blocks", ctypes.c_int32),
                ("gemv_lanes_per_row", ctypes.c_int32), ("gemv_splits", ctypes.c_int32),
                ("gemm_plan", ctypes.c_int32), ("gemv_split_combine", ctypes.c_int32)]


def make_force(gemv_kernel: str = "auto", gemv_plan: tuple | None = None, gemv_splits: int = 0,
               gemm_plan: str = "auto", gemv_split_combine: int = 0) -> Force:
    """An rfp4_force from names: gemv_kernel in GEMV_KERNEL, gemv_plan = (blocks per lane
    unit, lanes per row) of the dot-product kernel, gemv_splits of the tile kernel,
    gemm_plan in GEMM_PLAN, gemv_split_combine (1: the split tiles' parts combine without
    the last part's polling)."""
    p, cl = gemv_plan if gemv_plan is not None else (0, 0)
    return Force(GEMV_KERNEL[gemv_kernel], p, cl, gemv_splits, GEMM_PLAN[gemm_plan], gemv_split_combine)


class Rfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({rfp4_status_string(status)})")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load librfp4.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m gemm_rfp4_block_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    L = ctypes.CDLL(_LIB_PATH)
    c_i64, c_int, c_vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    L.rfp4_block_bytes.argtypes = [c_int]
    L.rfp4_block_bytes.restype = ctypes.c_size_t
    L.rfp4_row_bytes.argtypes = [c_int, c_i64]
    L.rfp4_row_bytes.restype = c_i64
    L.rfp4_status_string.argtypes = [c_int]
    L.rfp4_status_string.restype = ctypes.c_char_p
    L.rfp4_validate.argtypes = [c_vp, c_int, c_i64, c_i64, ctypes.POINTER(c_i64)]
    L.rfp4_validate.restype = c_int
    L.rfp4_dequant.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_vp]
    L.rfp4_dequant.restype = c_int
    L.rfp4_gemv.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_vp]
    L.rfp4_gemv.restype = c_int
    L.rfp4_gemv_multi.argtypes = [c_int, ctypes.POINTER(c_vp), ctypes.POINTER(c_i64), c_int, c_i64, c_vp,
                                  c_int, c_i64, c_i64, ctypes.POINTER(c_vp), ctypes.POINTER(c_i64), c_vp]
    L.rfp4_gemv_multi.restype = c_int
    L.rfp4_gemm.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp]
    L.rfp4_gemm.restype = c_int
    fp = ctypes.POINTER(Force)
    L.rfp4_gemv_multi_ex.argtypes = [c_int, ctypes.POINTER(c_vp), ctypes.POINTER(c_i64), c_int, c_i64, c_vp,
                                     c_int, c_i64, c_i64, ctypes.POINTER(c_vp), ctypes.POINTER(c_i64), fp, c_vp]
    L.rfp4_gemv_multi_ex.restype = c_int
    L.rfp4_gemm_ex.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, fp, c_vp]
    L.rfp4_gemm_ex.restype = c_int
    L.rfp4_gemm_noalloc.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, fp, c_vp]
    L.rfp4_gemm_noalloc.restype = c_int
    L.rfp4_dequant_bf16.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_vp]
    L.rfp4_dequant_bf16.restype = c_int
    L.rfp4_gemm_dequant.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]
    L.rfp4_gemm_dequant.restype = c_int
    L.rfp4_quantize.argtypes = [c_vp, c_int, c_i64, c_i64, c_i64, c_int, c_vp, c_vp]
    L.rfp4_quantize.restype = c_int
    _lib = L
    return L


def rfp4_block_bytes(layout: int) -> int:
    return int(lib().rfp4_block_bytes(layout))


def rfp4_row_bytes(layout: int, k: int) -> int:
    return int(lib().rfp4_row_bytes(layout, k))


def rfp4_status_string(status: int) -> str:
    return lib().rfp4_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != RFP4_OK:
        raise Rfp4Error(status, where)


def _stream(stream):
    import torch

    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _xdtype(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return RFP4_F16
    if t.dtype == torch.bfloat16:
        return RFP4_BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def rfp4_validate(w_host, layout: int, n: int, k: int):
    """Host-side row validation. ``w_host``: CPU uint8 numpy array or torch tensor,
    contiguous. Returns (status, first_bad_block)."""
    import numpy as np

    if hasattr(w_host, "numpy"):
        w_host = w_host.numpy()
    arr = np.ascontiguousarray(w_host, dtype=np.uint8)
    bad = ctypes.c_int64(-1)
    st = lib().rfp4_validate(arr.ctypes.data_as(ctypes.c_void_p), layout, n, k, ctypes.byref(bad))
    return int(st), int(bad.value)


def rfp4_dequant(w, layout: int, n: int, k: int, out=None, ldo: int | None = None, stream=None):
    """Dequantize device weights ``w`` (uint8, n x row_bytes) into fp32 ``out`` (n x ldo)."""
    import torch

    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    if ldo is None:
        ldo = out.stride(0) if out.dim() == 2 else k
    _check(lib().rfp4_dequant(_ptr(w), layout, n, k, _ptr(out), ldo, _stream(stream)), "rfp4_dequant")
    return out


def rfp4_dequant_bf16(w, layout: int, n: int, k: int, out=None, stream=None):
    """W as an (n, k) bf16 device tensor (bit-exact)."""
    import torch

    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=w.device)
    _check(lib().rfp4_dequant_bf16(_ptr(w), layout, n, k, _ptr(out), out.stride(0), _stream(stream)),
           "rfp4_dequant_bf16")
    return out


def rfp4_gemv(w, layout: int, n: int, k: int, x, y=None, stream=None, force: Force | None = None):
    """y[b, r] = sum_c W[r, c] x[b, c]; ``x`` (batch, >= k) f16/bf16 on the device, y fp32
    (batch, >= n). With ``force`` the call goes to rfp4_gemv_multi_ex."""
    import torch

    if x.dim() == 1:
        x = x.unsqueeze(0)
    batch = x.shape[0]
    if y is None:
        y = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    ldx = x.stride(0) if batch > 1 else max(k, x.stride(0))
    ldy = y.stride(0) if y.dim() == 2 and batch > 1 else max(n, y.stride(0) if y.dim() == 2 else n)
    if force is None:
        _check(lib().rfp4_gemv(_ptr(w), layout, n, k, _ptr(x), _xdtype(x), batch, ldx, _ptr(y), ldy,
                               _stream(stream)), "rfp4_gemv")
    else:
        rfp4_gemv_multi([w], layout, [n], k, x, [y], stream=stream, force=force, _ldy=[ldy])
    return y


def rfp4_gemv_multi(ws, layout: int, ns, k: int, x, ys=None, stream=None, force: Force | None = None,
                    _ldy=None):
    """One launch of len(ws) matvecs sharing x: ys[i][b, r] = sum_c Ws[i][r, c] x[b, c]."""
    import torch

    if x.dim() == 1:
        x = x.unsqueeze(0)
    batch = x.shape[0]
    count = len(ws)
    if ys is None:
        ys = [torch.empty((batch, int(n)), dtype=torch.float32, device=x.device) for n in ns]
    ldx = x.stride(0) if batch > 1 else max(k, x.stride(0))
    ldy = _ldy if _ldy is not None else [y.stride(0) if batch > 1 else max(int(n), y.stride(0))
                                         for y, n in zip(ys, ns)]
    wa = (ctypes.c_void_p * count)(*[w.data_ptr() for w in ws])
    na = (ctypes.c_int64 * count)(*[int(n) for n in ns])
    ya = (ctypes.c_void_p * count)(*[y.data_ptr() for y in ys])
    la = (ctypes.c_int64 * count)(*ldy)
    if force is None:
        _check(lib().rfp4_gemv_multi(count, wa, na, layout, k, _ptr(x), _xdtype(x), batch, ldx, ya, la,
                                     _stream(stream)), "rfp4_gemv_multi")
    else:
        _check(lib().rfp4_gemv_multi_ex(count, wa, na, layout, k, _ptr(x), _xdtype(x), batch, ldx, ya, la,
                                        ctypes.byref(force), _stream(stream)), "rfp4_gemv_multi_ex")
    return ys


def rfp4_gemm(w, layout: int, n: int, k: int, a, c=None, stream=None, force: Force | None = None):
    """C = A W^T with A (m, k) bf16 and C (m, n) bf16 on the device. With ``force`` the
    call goes to rfp4_gemm_ex."""
    import torch

    m = a.shape[0]
    if c is None:
        c = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if force is None:
        _check(lib().rfp4_gemm(_ptr(w), layout, n, k, _ptr(a), m, a.stride(0), _ptr(c), c.stride(0),
                               _stream(stream)), "rfp4_gemm")
    else:
        _check(lib().rfp4_gemm_ex(_ptr(w), layout, n, k, _ptr(a), m, a.stride(0), _ptr(c), c.stride(0),
                                  ctypes.byref(force), _stream(stream)), "rfp4_gemm_ex")
    return c


def rfp4_gemm_noalloc(w, layout: int, n: int, k: int, a, c, stream=None, force: Force | None = None):
    """C = A W^T like rfp4_gemm, with split plans' partial sums in the library's static
    per-GPU scratch array (no allocation); ``c`` (m, n) bf16 must be given."""
    m = a.shape[0]
    _check(lib().rfp4_gemm_noalloc(_ptr(w), layout, n, k, _ptr(a), m, a.stride(0), _ptr(c), c.stride(0),
                                   ctypes.byref(force) if force is not None else None, _stream(stream)),
           "rfp4_gemm_noalloc")
    return c


def rfp4_gemm_dequant(w, layout: int, n: int, k: int, a, wbuf=None, c=None, stream=None):
    """C = A W^T computed as bf16 dequantization into ``wbuf`` (n, k) plus a dense bf16
    GEMM (rocBLAS)."""
    import torch

    m = a.shape[0]
    if c is None:
        c = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if wbuf is None:
        wbuf = torch.empty((n, k), dtype=torch.bfloat16, device=a.device)
    _check(lib().rfp4_gemm_dequant(_ptr(w), layout, n, k, _ptr(a), m, a.stride(0), _ptr(c), c.stride(0),
                                   _ptr(wbuf), wbuf.stride(0), _stream(stream)), "rfp4_gemm_dequant")
    return c


def rfp4_quantize(src, layout: int, out=None, stream=None):
    """Encode ``src`` (n, k) float32/bfloat16/float16 on the device into packed rows
    (uint8 tensor of shape (n, row_bytes))."""
    import torch

    codes = {torch.float32: RFP4_F32, torch.bfloat16: RFP4_BF16, torch.float16: RFP4_F16}
    if src.dtype not in codes:
        raise TypeError(f"src must be float32, bfloat16 or float16, got {src.dtype}")
    n, k = src.shape
    if src.stride(1) != 1:
        raise ValueError("src rows must be contiguous")
    if out is None:
        out = torch.empty((n, max(rfp4_row_bytes(layout, k), 0)), dtype=torch.uint8, device=src.device)
    _check(lib().rfp4_quantize(_ptr(src), codes[src.dtype], n, k, src.stride(0), layout, _ptr(out),
                               _stream(stream)), "rfp4_quantize")
    return out


__all__ = [
    "RFP4_DUAL", "RFP4_FAST", "RFP4_F16", "RFP4_BF16", "Rfp4Error", "lib", "library_path",
    "rfp4_block_bytes", "rfp4_row_bytes", "rfp4_status_string", "rfp4_validate",
    "rfp4_dequant", "rfp4_dequant_bf16", "rfp4_gemv", "rfp4_gemv_multi", "rfp4_gemm",
    "rfp4_gemm_dequant", "rfp4_quantize", "RFP4_F32", "MAX_GEMV_PARTS", "Force", "make_force",
    "GEMV_KERNEL", "GEMM_PLAN", "rfp4_gemm_noalloc", "RFP4_ERR_SCRATCH", "GEMM_SCRATCH_BYTES",
]
