"""GPU parity on seeded random shapes: every entry point against the fp64 CPU oracle.

Shapes, layouts, activation dtypes, padded leading dimensions and the forced kernel or
plan are drawn per case from a generator seeded with the case index, so a failing case
is reproduced by its id alone. Sizes stay small enough for the oracle (GEMM up to
300 x 400 x 3200); they cross tile edges, ragged rows, odd block counts and every
batch. Acceptance as in test_gpu_parity: bit- or byte-exact for dequantization and
encoding, max |y - y_ref| / sum |w x| <= 2e-3 for the contractions.
"""

import numpy as np
import pytest
import torch

import gemm_rfp4_block_amd as R
import oracle.rfp4_oracle as O
import synth
from tests.abi_calls import gemm_raw, gemv_raw
from tests.test_gpu_parity import gemm_error

pytestmark = pytest.mark.gpu
TOL = 2e-3
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x64(t):
    return t.to(torch.float64).cpu().numpy()


def log_uniform(rng, lo, hi):
    return int(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))))


def round8(v):
    return (v + 7) // 8 * 8


@pytest.mark.parametrize("case", range(40), ids=lambda i: f"gemv{i}")
def test_random_gemv(case):
    rng = np.random.default_rng(71000 + case)
    layout = int(rng.integers(0, 2))
    n = log_uniform(rng, 1, 400)
    k = 32 * log_uniform(rng, 1, 300)
    batch = int(rng.integers(1, 9))
    dt = ("f16", "bf16")[int(rng.integers(0, 2))]
    mode = (None, "dot", "tiles")[int(rng.integers(0, 3))]
    f = R.make_force(mode) if mode is not None else None
    ldx = k + (0, 8, 24)[int(rng.integers(0, 3))]
    ldy = n + (0, 3)[int(rng.integers(0, 2))]
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, batch, k, dt)
    xd = torch.zeros((batch, ldx), dtype=x.dtype, device=DEV)
    xd[:, :k] = x.to(DEV)
    y = torch.full((batch, ldy), float("nan"), dtype=torch.float32, device=DEV)
    st = gemv_raw(dev(w), layout, n, k, xd, batch, ldx, y, ldy, force=f)
    assert st == R.RFP4_OK, R.rfp4_status_string(st)
    torch.cuda.synchronize()
    out = y.cpu().numpy()
    assert np.all(np.isnan(out[:, n:])), "gemv wrote past n"
    y_ref, den = O.gemv(w, layout, n, k, x64(x))
    assert O.normalized_error(out[:, :n], y_ref, den) <= TOL


GEMM_PLANS = (None, "main", "tail", "tail2", "tail4", "msplit2", "msplit3", "nosplit")


@pytest.mark.parametrize("case", range(24), ids=lambda i: f"gemm{i}")
def test_random_gemm(case):
    rng = np.random.default_rng(72000 + case)
    layout = int(rng.integers(0, 2))
    m = log_uniform(rng, 1, 300)
    n = log_uniform(rng, 1, 400)
    k = 32 * log_uniform(rng, 1, 100)
    plan = GEMM_PLANS[int(rng.integers(0, len(GEMM_PLANS)))]
    f = R.make_force(gemm_plan=plan) if plan is not None else None
    ldc = round8(n) + 8
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    a = synth.activations(rng, m, k, "bf16")
    c = torch.full((m, ldc), float("nan"), dtype=torch.bfloat16, device=DEV)
    ad = a.to(DEV).contiguous()
    st = gemm_raw(dev(w), layout, n, k, ad, m, k, c, ldc, force=f)
    assert st == R.RFP4_OK, R.rfp4_status_string(st)
    torch.cuda.synchronize()
    out = c.to(torch.float64).cpu().numpy()
    assert np.all(np.isnan(out[:, n:])), "gemm wrote past n"
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(out[:, :n], c_ref, den) <= TOL


@pytest.mark.parametrize("case", range(16), ids=lambda i: f"dequant{i}")
def test_random_dequant(case):
    rng = np.random.default_rng(73000 + case)
    layout = int(rng.integers(0, 2))
    n = log_uniform(rng, 1, 300)
    k = 32 * log_uniform(rng, 1, 300)
    w = synth.weights(rng, layout, n, k, stress_frac=0.05)
    got = R.rfp4_dequant(dev(w), layout, n, k).cpu().numpy()
    want = O.dequantize_f32(w, layout, n, k)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("case", range(16), ids=lambda i: f"quantize{i}")
def test_random_quantize(case):
    rng = np.random.default_rng(74000 + case)
    layout = int(rng.integers(0, 2))
    n = log_uniform(rng, 1, 300)
    k = 32 * log_uniform(rng, 1, 200)
    dt = ("f32", "bf16", "f16")[int(rng.integers(0, 3))]
    src = synth.real_weights(rng, n, k, dt)
    got = R.rfp4_quantize(src.to(DEV), layout).cpu().numpy()
    want = O.quantize(src.double().numpy(), layout)
    assert np.array_equal(got, want)
