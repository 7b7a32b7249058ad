"""C-ABI boundary tests that need no GPU.

The library must load on a machine without a GPU, export every function that
include/rfp4.h declares, and reject bad arguments before making any HIP call (so
every call below carries at least one invalid argument and never launches a kernel).
Host-side row validation is compared with the oracle's.
"""

import ctypes
import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import gemm_rfp4_block_amd as R
import oracle.rfp4_oracle as O
import synth
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "rfp4.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(R.library_path()):
        from gemm_rfp4_block_amd.build import build

        build()
    return R.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"RFP4_API\s+[\w\s\*]+?\b(rfp4_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(R.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", R.library_path()], capture_output=True, text=True)
    exported = set(re.findall(r" T (rfp4_\w+)", out.stdout))
    assert exported == set(declared_functions())


BENCH_HEADER = os.path.join(ROOT, "include", "rfp4_bench.h")
BENCH_LIB = os.path.join(ROOT, "gemm_rfp4_block_amd", "_lib", "librfp4_bench.so")


def test_bench_library_exports_its_header_and_checks_arguments(L):
    """librfp4_bench.so (the read and matrix-core ceilings of the benchmark) exports
    exactly what include/rfp4_bench.h declares and rejects bad arguments before any HIP
    call (-1), so this runs without a GPU."""
    declared = sorted(set(re.findall(r"\b(rfp4bench_\w+)\s*\(", open(BENCH_HEADER).read())))
    assert declared == ["rfp4bench_mfma", "rfp4bench_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", BENCH_LIB], capture_output=True, text=True)
    assert set(re.findall(r" T (rfp4bench_\w+)", out.stdout)) == set(declared)
    B = ctypes.CDLL(BENCH_LIB)
    B.rfp4bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    B.rfp4bench_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = ctypes.c_void_p(0x10000)
    for p, nbytes, unroll, wgs, snk in ((None, 64, 1, 8, sink), (0x10000, 0, 1, 8, sink), (0x10000, 24, 1, 8, sink),
                                        (0x10008, 64, 1, 8, sink), (0x10000, 64, 3, 8, sink),
                                        (0x10000, 64, 1, 0, sink), (0x10000, 64, 1, 33, sink),
                                        (0x10000, 64, 1, 8, None)):
        assert B.rfp4bench_read(p, nbytes, unroll, wgs, snk, None) == -1
    for wgs, threads, iters, snk in ((0, 256, 1, sink), (9, 256, 1, sink), (1, 192, 1, sink), (1, 1024, 1, sink),
                                     (1, 256, 0, sink), (1, 256, 1, None)):
        assert B.rfp4bench_mfma(wgs, threads, iters, snk, None) == -1


def test_block_and_row_bytes(L):
    assert R.rfp4_block_bytes(R.RFP4_DUAL) == O.block_bytes(O.DUAL) == 18
    assert R.rfp4_block_bytes(R.RFP4_FAST) == O.block_bytes(O.FAST) == 17
    assert R.rfp4_block_bytes(7) == 0
    for k in (32, 512, 5120, 17408):
        assert R.rfp4_row_bytes(R.RFP4_DUAL, k) == O.row_bytes(O.DUAL, k)
        assert R.rfp4_row_bytes(R.RFP4_FAST, k) == O.row_bytes(O.FAST, k)
    assert R.rfp4_row_bytes(R.RFP4_DUAL, 33) == -1
    assert R.rfp4_row_bytes(R.RFP4_DUAL, 0) == -1
    assert R.rfp4_row_bytes(5, 64) == -1


def test_status_strings(L):
    for st in range(7):
        assert R.rfp4_status_string(st)
    assert R.rfp4_status_string(99) == "unknown status"


# Fake, 16-byte aligned "device" addresses. Every call below fails an argument check
# first, so these are never dereferenced or handed to HIP.
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
NULL = ctypes.c_void_p(0)
UNALIGNED = ctypes.c_void_p(0x10008)  # breaks W's and the dequant outputs' 16-byte rule
ODD2 = ctypes.c_void_p(0x10002)  # breaks the 4-byte rule of x, y, A and C


def test_dequant_argument_errors(L):
    f = L.rfp4_dequant
    assert f(NULL, 0, 4, 512, P2, 512, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 4, 512, NULL, 512, NULL) == R.RFP4_ERR_NULL
    assert f(P, 2, 4, 512, P2, 512, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(P, 0, 0, 512, P2, 512, NULL) == R.RFP4_ERR_SHAPE
    assert f(P, 0, 4, 500, P2, 512, NULL) == R.RFP4_ERR_SHAPE
    assert f(P, 0, 4, 0, P2, 512, NULL) == R.RFP4_ERR_SHAPE
    assert f(P, 0, 4, 512, P2, 511, NULL) == R.RFP4_ERR_SHAPE  # ldo < k
    # rows of any length are accepted (k = 96: 54-byte rows); the other checks still apply
    assert f(P, 0, 4, 96, P2, 95, NULL) == R.RFP4_ERR_SHAPE  # ldo < k
    assert f(UNALIGNED, 1, 4, 96, P2, 96, NULL) == R.RFP4_ERR_UNSUPPORTED  # W base
    assert f(P, 0, 1 << 30, 1 << 20, P2, 1 << 20, NULL) == R.RFP4_ERR_SHAPE  # W > 2^40 bytes
    assert f(UNALIGNED, 0, 4, 512, P2, 512, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(P, 0, 4, 512, UNALIGNED, 512, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(P, 0, 4, 512, P2, 514, NULL) == R.RFP4_ERR_UNSUPPORTED  # ldo % 4


def test_gemv_argument_errors(L):
    f = L.rfp4_gemv
    assert f(NULL, 0, 8, 512, P2, 0, 1, 512, P, 8, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 8, 512, NULL, 0, 1, 512, P, 8, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 8, 512, P2, 0, 1, 512, NULL, 8, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 8, 512, P2, 2, 1, 512, P, 8, NULL) == R.RFP4_ERR_UNSUPPORTED  # dtype
    assert f(P, 3, 8, 512, P2, 0, 1, 512, P, 8, NULL) == R.RFP4_ERR_UNSUPPORTED  # layout
    assert f(P, 0, 8, 512, P2, 0, 0, 512, P, 8, NULL) == R.RFP4_ERR_SHAPE  # batch 0
    assert f(P, 0, 8, 512, P2, 0, 9, 512, P, 8, NULL) == R.RFP4_ERR_SHAPE  # batch 9
    assert f(P, 0, 8, 512, P2, 0, 1, 500, P, 8, NULL) == R.RFP4_ERR_SHAPE  # ldx < k
    assert f(P, 0, 8, 512, P2, 0, 1, 512, P, 7, NULL) == R.RFP4_ERR_SHAPE  # ldy < n
    assert f(P, 0, -1, 512, P2, 0, 1, 512, P, 8, NULL) == R.RFP4_ERR_SHAPE
    assert f(P, 0, 8, 2**31, P2, 0, 1, 2**31, P, 8, NULL) == R.RFP4_ERR_SHAPE
    assert f(P, 0, 8, 512, P2, 0, 2, 517, P, 8, NULL) == R.RFP4_ERR_UNSUPPORTED  # ldx odd
    assert f(P, 0, 8, 512, ODD2, 0, 1, 512, P, 8, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(P, 0, 8, 512, P2, 0, 1, 512, ODD2, 8, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(UNALIGNED, 1, 8, 96, P2, 0, 1, 96, P, 8, NULL) == R.RFP4_ERR_UNSUPPORTED  # W base
    assert f(P, 1, 8, 96, P2, 0, 1, 95, P, 8, NULL) == R.RFP4_ERR_SHAPE  # ldx < k, 51-byte rows


def test_gemv_multi_argument_errors(L):
    import ctypes

    f = L.rfp4_gemv_multi

    def arr(t, vals):
        return (t * len(vals))(*vals)

    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    w2 = arr(vp, [P, P])
    n2 = arr(i64, [8, 16])
    y2 = arr(vp, [P, P])
    l2 = arr(i64, [8, 16])
    assert f(0, w2, n2, 0, 512, P2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_SHAPE  # count 0
    assert f(R.MAX_GEMV_PARTS + 1, w2, n2, 0, 512, P2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_SHAPE
    assert f(2, None, n2, 0, 512, P2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_NULL
    assert f(2, w2, None, 0, 512, P2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_NULL
    assert f(2, w2, n2, 0, 512, P2, 0, 1, 512, None, l2, NULL) == R.RFP4_ERR_NULL
    assert f(2, w2, n2, 0, 512, P2, 0, 1, 512, y2, None, NULL) == R.RFP4_ERR_NULL
    # one bad part is reported with that part's error
    assert f(2, arr(vp, [P, NULL]), n2, 0, 512, P2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_NULL
    assert f(2, w2, arr(i64, [8, 0]), 0, 512, P2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_SHAPE
    assert f(2, w2, n2, 0, 512, P2, 0, 1, 512, arr(vp, [P, ODD2]), l2, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(2, w2, n2, 0, 512, P2, 0, 1, 512, y2, arr(i64, [8, 15]), NULL) == R.RFP4_ERR_SHAPE
    assert f(2, arr(vp, [P, UNALIGNED]), n2, 0, 512, P2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_UNSUPPORTED
    # the total row count must fit in 2^31 - 1
    big = 2**31 - 16
    assert f(2, w2, arr(i64, [big, 32]), 0, 512, P2, 0, 1, 512, y2, arr(i64, [big, 32]), NULL) == R.RFP4_ERR_SHAPE
    # shared arguments are checked as in rfp4_gemv
    assert f(2, w2, n2, 0, 512, P2, 2, 1, 512, y2, l2, NULL) == R.RFP4_ERR_UNSUPPORTED  # dtype
    assert f(2, w2, n2, 0, 512, P2, 0, 9, 512, y2, l2, NULL) == R.RFP4_ERR_SHAPE  # batch
    assert f(2, w2, n2, 0, 512, NULL, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_NULL  # x
    assert f(2, w2, n2, 0, 512, ODD2, 0, 1, 512, y2, l2, NULL) == R.RFP4_ERR_UNSUPPORTED


def test_dequant_bf16_argument_errors(L):
    f = L.rfp4_dequant_bf16
    assert f(NULL, 0, 8, 512, P, 512, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 8, 512, NULL, 512, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 8, 512, P, 511, NULL) == R.RFP4_ERR_SHAPE  # ldo < k
    assert f(P, 0, 8, 512, P, 516, NULL) == R.RFP4_ERR_UNSUPPORTED  # ldo % 8
    assert f(P, 0, 8, 512, UNALIGNED, 512, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(P, 5, 8, 512, P, 512, NULL) == R.RFP4_ERR_UNSUPPORTED  # layout
    assert f(P, 0, 8, 500, P, 512, NULL) == R.RFP4_ERR_SHAPE  # k % 32
    assert f(P, 0, 2**20, 512, P, 2**20, NULL) == R.RFP4_ERR_SHAPE  # n * ldo > 2^39


def test_gemm_dequant_argument_errors(L):
    f = L.rfp4_gemm_dequant
    ok = (P, 0, 64, 512, P2, 16, 512, P, 64)
    assert f(*ok, NULL, 512, NULL) == R.RFP4_ERR_NULL  # wbuf
    assert f(*ok, P2, 511, NULL) == R.RFP4_ERR_SHAPE  # ldw < k
    assert f(*ok, P2, 520 + 4, NULL) == R.RFP4_ERR_UNSUPPORTED  # ldw % 8
    assert f(*ok, UNALIGNED, 512, NULL) == R.RFP4_ERR_UNSUPPORTED
    # the GEMM arguments are checked as in rfp4_gemm, before wbuf
    assert f(NULL, 0, 64, 512, P2, 16, 512, P, 64, NULL, 512, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 64, 512, P2, 0, 512, P, 64, P2, 512, NULL) == R.RFP4_ERR_SHAPE  # m = 0
    assert f(P, 0, 64, 512, P2, 16, 512, P, 63, P2, 512, NULL) == R.RFP4_ERR_SHAPE  # ldc < n
    assert f(P, 0, 64, 512, P2, 16, 517, P, 64, P2, 512, NULL) == R.RFP4_ERR_UNSUPPORTED  # lda odd


def test_gemm_argument_errors(L):
    f = L.rfp4_gemm
    assert f(NULL, 0, 64, 512, P2, 16, 512, P, 64, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 64, 512, NULL, 16, 512, P, 64, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 64, 512, P2, 16, 512, NULL, 64, NULL) == R.RFP4_ERR_NULL
    assert f(P, 0, 64, 512, P2, 0, 512, P, 64, NULL) == R.RFP4_ERR_SHAPE  # m = 0
    assert f(P, 0, 64, 512, P2, 16, 511, P, 64, NULL) == R.RFP4_ERR_SHAPE  # lda < k
    assert f(P, 0, 64, 512, P2, 16, 512, P, 63, NULL) == R.RFP4_ERR_SHAPE  # ldc < n
    assert f(P, 0, 64, 512, P2, 16, 520, ODD2, 68, NULL) == R.RFP4_ERR_UNSUPPORTED  # C base
    assert f(P, 0, 64, 512, ODD2, 16, 520, P, 68, NULL) == R.RFP4_ERR_UNSUPPORTED  # A base
    assert f(P, 0, 64, 512, P2, 16, 517, P, 64, NULL) == R.RFP4_ERR_UNSUPPORTED  # lda odd
    assert f(P, 4, 64, 512, P2, 16, 512, P, 64, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(UNALIGNED, 0, 64, 96, P2, 16, 96, P, 64, NULL) == R.RFP4_ERR_UNSUPPORTED  # W base
    assert f(P, 0, 64, 96, P2, 16, 95, P, 64, NULL) == R.RFP4_ERR_SHAPE  # lda < k, 54-byte rows


BAD_FORCES = [  # each field outside the values include/rfp4.h lists
    dict(gemv_kernel=5), dict(gemv_kernel=-1), dict(gemv_unit_blocks=3, gemv_lanes_per_row=16),
    dict(gemv_unit_blocks=1, gemv_lanes_per_row=12), dict(gemv_unit_blocks=2, gemv_lanes_per_row=128),
    dict(gemv_unit_blocks=1, gemv_lanes_per_row=0), dict(gemv_unit_blocks=0, gemv_lanes_per_row=8),
    dict(gemv_splits=5), dict(gemv_splits=-1), dict(gemm_plan=9), dict(gemm_plan=-2),
    dict(gemv_split_combine=2), dict(gemv_split_combine=-1),
]


@pytest.mark.parametrize("bad", BAD_FORCES, ids=lambda d: "-".join(f"{k}{v}" for k, v in d.items()))
def test_force_fields_checked_before_any_hip_call(L, bad):
    f = R.Force(**bad)
    one = (ctypes.c_void_p * 1)(0x10000)
    n1 = (ctypes.c_int64 * 1)(8)
    y1 = (ctypes.c_void_p * 1)(0x20000)
    ld = (ctypes.c_int64 * 1)(8)
    assert L.rfp4_gemv_multi_ex(1, one, n1, 0, 512, P2, 0, 1, 512, y1, ld, ctypes.byref(f), NULL) == \
        R.RFP4_ERR_UNSUPPORTED
    assert L.rfp4_gemm_ex(P, 0, 64, 512, P2, 16, 512, P, 64, ctypes.byref(f), NULL) == R.RFP4_ERR_UNSUPPORTED


def test_force_entry_points_check_shapes(L):
    """A valid (or NULL) force leaves the ordinary argument checks in place."""
    f = R.make_force("tiles", gemv_splits=2, gemm_plan="tail4")
    one = (ctypes.c_void_p * 1)(0x10000)
    n1 = (ctypes.c_int64 * 1)(8)
    y1 = (ctypes.c_void_p * 1)(0x20000)
    ld = (ctypes.c_int64 * 1)(8)
    for fp in (ctypes.byref(f), None):
        assert L.rfp4_gemv_multi_ex(1, one, n1, 0, 512, P2, 0, 9, 512, y1, ld, fp, NULL) == R.RFP4_ERR_SHAPE
        assert L.rfp4_gemv_multi_ex(1, one, n1, 0, 512, NULL, 0, 1, 512, y1, ld, fp, NULL) == R.RFP4_ERR_NULL
        assert L.rfp4_gemm_ex(P, 0, 64, 512, P2, 16, 511, P, 64, fp, NULL) == R.RFP4_ERR_SHAPE
        assert L.rfp4_gemm_ex(P, 0, 64, 512, P2, 16, 512, ODD2, 64, fp, NULL) == R.RFP4_ERR_UNSUPPORTED


def test_library_sources_read_no_environment_and_never_free_or_synchronize():
    """The product path takes no hidden inputs (no getenv) and never frees memory or
    synchronizes a stream or the device inside a call."""
    csrc = os.path.join(ROOT, "gemm_rfp4_block_amd", "csrc")
    banned = re.compile(r"\b(getenv|secure_getenv|hipFree|hipFreeAsync|hipStreamSynchronize|"
                        r"hipDeviceSynchronize|hipEventSynchronize)\s*\(")
    for name in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, name)).read()
        code = re.sub(r"//[^\n]*", "", text)  # comments may name them
        assert not banned.search(code), name


def test_quantize_argument_errors(L):
    f = L.rfp4_quantize
    assert f(P, 3, 4, 64, 64, 0, P2, NULL) == R.RFP4_ERR_UNSUPPORTED  # dtype
    assert f(P, R.RFP4_BF16, 4, 64, 64, 2, P2, NULL) == R.RFP4_ERR_UNSUPPORTED  # layout
    assert f(P, R.RFP4_BF16, 0, 64, 64, 0, P2, NULL) == R.RFP4_ERR_SHAPE  # n = 0
    assert f(P, R.RFP4_BF16, 4, 48, 48, 0, P2, NULL) == R.RFP4_ERR_SHAPE  # k % 32
    assert f(P, R.RFP4_BF16, 4, 64, 56, 0, P2, NULL) == R.RFP4_ERR_SHAPE  # lds < k
    assert f(P, R.RFP4_BF16, 1 << 20, 64, 1 << 20, 0, P2, NULL) == R.RFP4_ERR_SHAPE  # n * lds > 2^39
    assert f(NULL, R.RFP4_BF16, 4, 64, 64, 0, P2, NULL) == R.RFP4_ERR_NULL
    assert f(P, R.RFP4_BF16, 4, 64, 64, 0, NULL, NULL) == R.RFP4_ERR_NULL
    assert f(UNALIGNED, R.RFP4_BF16, 4, 64, 64, 0, P2, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(P, R.RFP4_BF16, 4, 64, 64, 0, UNALIGNED, NULL) == R.RFP4_ERR_UNSUPPORTED
    assert f(P, R.RFP4_BF16, 4, 64, 68, 0, P2, NULL) == R.RFP4_ERR_UNSUPPORTED  # 136-byte rows
    assert f(P, R.RFP4_F32, 4, 64, 66, 1, P2, NULL) == R.RFP4_ERR_UNSUPPORTED  # 264-byte rows


def test_validate_null_and_shape(L):
    bad = ctypes.c_int64(123)
    assert L.rfp4_validate(NULL, 0, 1, 32, ctypes.byref(bad)) == R.RFP4_ERR_NULL
    assert bad.value == -1
    buf = (ctypes.c_uint8 * 18)()
    assert L.rfp4_validate(buf, 0, 1, 31, None) == R.RFP4_ERR_SHAPE
    assert L.rfp4_validate(buf, 9, 1, 32, None) == R.RFP4_ERR_UNSUPPORTED
    assert L.rfp4_validate(buf, 0, 1, 32, None) == R.RFP4_OK


@pytest.mark.parametrize("layout", [0, 1])
def test_validate_matches_oracle(L, layout):
    rng = np.random.default_rng(11 + layout)
    n, k = 24, 1024
    w = synth.weights(rng, layout, n, k)
    assert R.rfp4_validate(w, layout, n, k) == (R.RFP4_OK, -1)
    assert O.validate(w, layout, n, k) == (True, -1)
    bb = synth.block_bytes(layout)
    nb = k // 32
    for trial in range(20):
        wb = w.reshape(n, nb, bb).copy()
        cnt = int(rng.integers(1, 4))
        for _ in range(cnt):
            r, j = int(rng.integers(0, n)), int(rng.integers(0, nb))
            s = int(rng.integers(16, bb))
            wb[r, j, s] = 0x7F | (int(rng.integers(0, 2)) << 7)
        wb[:, :, :16] |= 0x7F  # index bytes never count
        flat = wb.reshape(n, -1)
        ok, first = O.validate(flat, layout, n, k)
        st, bad = R.rfp4_validate(flat, layout, n, k)
        assert not ok
        assert st == R.RFP4_ERR_NONFINITE_SCALE and bad == first


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for several, it prints one JSON line naming the
    reason and exits with status 2 before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
