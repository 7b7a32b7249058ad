"""Activations and outputs at 4-byte (not 16-byte) alignment, through every contraction
kernel, on the C ABI.

The boundary accepts x, y, A and C on 4-byte boundaries, with even leading dimensions
for x and A and any ldy and ldc. Here every such buffer starts 4 bytes past a fresh
allocation and the leading dimensions are k + 2 (x, A) and n + 1 (y, C), so no
activation or output row is 16-byte aligned. The same kernel and plan run as for the
aligned call (the choice depends on the shape only), so the results must equal the
aligned call's bit for bit, and the gaps between rows must stay untouched. The aligned
calls themselves are checked against the oracle by the other parity tests."""

import numpy as np
import pytest
import torch

import gemm_rfp4_block_amd as R
import synth
from tests.abi_calls import gemm_raw, gemv_raw

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

GEMV_CASES = [  # layout, n, k, batch, x dtype, forced kernel, tile-kernel splits
    (0, 1024, 5120, 1, "f16", "dot", 0),
    (1, 1024, 5120, 2, "bf16", "dot", 0),
    (0, 512, 17408, 1, "f16", "dot", 0),  # long rows: 1024-thread workgroups
    (0, 8192, 5120, 1, "f16", "tall", 0),
    (1, 1024, 6144, 4, "bf16", "tiles", 1),
    (1, 512, 17408, 8, "bf16", "tiles", 2),  # split tiles
    (0, 1000, 4128, 3, "f16", "auto", 0),  # ragged rows, k % 128 != 0
]


def offset_rows(rows, cols, ld, dtype, off_elems, fill):
    """(storage, view): a rows x cols view with row stride ld that starts off_elems
    elements into a fresh allocation filled with `fill`."""
    store = torch.full((rows * ld + off_elems,), fill, dtype=dtype, device=DEV)
    view = store[off_elems:off_elems + rows * ld].view(rows, ld)[:, :cols]
    return store, view


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "L{}n{}k{}b{}{}-{}-s{}".format(*c))
def test_gemv_four_byte_aligned_rows_equal_aligned_call(case):
    layout, n, k, batch, dt, kernel, splits = case
    w = synth.weights_device(layout, n, k, 7100 + n + k, DEV)
    x = synth.activations_device(batch, k, dt, 7200 + batch, DEV)
    force = R.make_force(kernel, gemv_splits=splits)
    y_ref = torch.empty((batch, n), dtype=torch.float32, device=DEV)
    assert gemv_raw(w, layout, n, k, x, batch, k, y_ref, n, force) == R.RFP4_OK

    ldx, ldy = k + 2, n + 1
    _, xv = offset_rows(batch, k, ldx, x.dtype, 2, 0.0)
    xv.copy_(x)
    y_store, yv = offset_rows(batch, n, ldy, torch.float32, 1, float("nan"))
    assert xv.data_ptr() % 16 == 4 and yv.data_ptr() % 16 == 4
    assert gemv_raw(w, layout, n, k, xv, batch, ldx, yv, ldy, force) == R.RFP4_OK
    torch.cuda.synchronize()
    assert torch.equal(yv, y_ref), f"max diff {float((yv - y_ref).abs().max())}"
    gaps = y_store[1:].view(batch, ldy)[:, n:]
    assert bool(torch.isnan(gaps).all()) and bool(torch.isnan(y_store[:1]).all())


GEMM_CASES = [  # m, n, k, plan
    (512, 1024, 5120, "main"),
    (512, 1024, 5120, "tail2"),
    (300, 1000, 5120, "msplit2"),
    (256, 768, 4128, "auto"),  # k tail
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "m{}n{}k{}-{}".format(*c))
def test_gemm_four_byte_aligned_rows_equal_aligned_call(case):
    m, n, k, plan = case
    layout = 0
    w = synth.weights_device(layout, n, k, 7300 + n, DEV)
    a = synth.activations_device(m, k, "bf16", 7400 + m, DEV)
    force = R.make_force(gemm_plan=plan)
    c_ref = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    assert gemm_raw(w, layout, n, k, a, m, k, c_ref, n, force) == R.RFP4_OK

    lda, ldc = k + 2, n + 1
    _, av = offset_rows(m, k, lda, torch.bfloat16, 2, 0.0)
    av.copy_(a)
    c_store, cv = offset_rows(m, n, ldc, torch.bfloat16, 2, float("nan"))
    assert av.data_ptr() % 16 == 4 and cv.data_ptr() % 16 == 4
    assert gemm_raw(w, layout, n, k, av, m, lda, cv, ldc, force) == R.RFP4_OK
    torch.cuda.synchronize()
    assert torch.equal(cv.float(), c_ref.float())
    gaps = c_store[2:].view(m, ldc)[:, n:]
    assert bool(torch.isnan(gaps.float()).all()) and bool(torch.isnan(c_store[:2].float()).all())


def test_gemm_noalloc_four_byte_aligned_rows_equal_aligned_call():
    m, n, k = 512, 1024, 5120
    w = synth.weights_device(0, n, k, 7500, DEV)
    a = synth.activations_device(m, k, "bf16", 7501, DEV)
    c_ref = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    R.rfp4_gemm_noalloc(w, 0, n, k, a, c_ref)
    _, av = offset_rows(m, k, k + 2, torch.bfloat16, 2, 0.0)
    av.copy_(a)
    _, cv = offset_rows(m, n, n + 1, torch.bfloat16, 2, float("nan"))
    R.rfp4_gemm_noalloc(w, 0, n, k, av, cv)
    torch.cuda.synchronize()
    assert torch.equal(cv.float(), c_ref.float())


def test_aligned_reference_matches_oracle_on_one_case():
    """The bitwise comparisons above lean on the aligned calls; tie one of them to the
    oracle here as well (full rows, normalized error within the 2e-3 bound)."""
    import oracle.rfp4_oracle as O

    layout, n, k, batch = 1, 256, 4128, 3
    w_host = synth.weights(np.random.default_rng(7600), layout, n, k)
    x = synth.activations_device(batch, k, "bf16", 7601, DEV)
    _, xv = offset_rows(batch, k, k + 2, x.dtype, 2, 0.0)
    xv.copy_(x)
    _, yv = offset_rows(batch, n, n + 1, torch.float32, 1, float("nan"))
    wd = torch.from_numpy(w_host).to(DEV)
    assert gemv_raw(wd, layout, n, k, xv, batch, k + 2, yv, n + 1) == R.RFP4_OK
    torch.cuda.synchronize()
    y_ref, den = O.gemv(w_host, layout, n, k, x.to(torch.float64).cpu().numpy())
    assert O.normalized_error(yv.cpu().numpy(), y_ref, den) <= 2e-3
