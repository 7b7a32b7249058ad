"""rfp4_gemm_noalloc (the GEMM for callers that cannot allocate) against rfp4_gemm_ex,
through the C ABI: two calls in a row, the second on a smaller input, each bit-identical
to the workspace entry point with the same plan; a shape whose default plan's partial
sums do not fit the static scratch array runs a plan that fits and stays within the
oracle's tolerance; a forced plan that needs more is rejected before any launch."""

import numpy as np
import pytest
import torch

import gemm_rfp4_block_amd as R
import oracle.rfp4_oracle as O
import synth
from tests.abi_calls import gemm_raw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


def noalloc(wd, layout, n, k, ad, c, force=None):
    f = R.make_force(**force) if force else None
    return R.lib().rfp4_gemm_noalloc(R._ptr(wd), layout, n, k, R._ptr(ad), ad.shape[0], ad.stride(0), R._ptr(c),
                                     c.stride(0), __import__("ctypes").byref(f) if f is not None else None,
                                     R._stream(None))


def gemm_error(c, c_ref, den):
    c = np.asarray(c, dtype=np.float64)
    mag = np.abs(c_ref)
    half_ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 8), 0.0)
    excess = np.maximum(np.abs(c - c_ref) - half_ulp, 0.0)
    return O.normalized_error(c_ref + np.sign(c - c_ref) * excess, c_ref, den)


CASES = [  # layout, m, n, k, forced plan: the prefill shape (its split tail, 16 MiB of
           # partial sums), then smaller inputs with split plans
    (0, 2048, 17408, 5120, None),
    (0, 300, 1040, 2048, "tail2"),
    (1, 130, 264, 1024, "msplit2"),
]


def test_noalloc_equals_gemm_two_calls_in_a_row():
    outs = []
    for layout, m, n, k, plan in CASES:
        rng = np.random.default_rng(15000 + m)
        wd = torch.from_numpy(synth.weights(rng, layout, n, k)).to(DEV)
        ad = synth.activations(rng, m, k, "bf16").to(DEV).contiguous()
        c1 = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
        c2 = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
        force = dict(gemm_plan=plan) if plan else None
        st = noalloc(wd, layout, n, k, ad, c1, force)
        assert st == R.RFP4_OK, R.rfp4_status_string(st)
        st = gemm_raw(wd, layout, n, k, ad, m, k, c2, n, force=R.make_force(**force) if force else None)
        assert st == R.RFP4_OK, R.rfp4_status_string(st)
        outs.append((c1, c2))
    torch.cuda.synchronize()
    for (c1, c2), case in zip(outs, CASES):
        assert torch.equal(c1.view(torch.int16), c2.view(torch.int16)), case


def test_noalloc_runs_a_plan_that_fits_the_scratch():
    """8192 x 17408 x 5120: rfp4_gemm's plan would keep 64 MiB of partial sums, more
    than the array holds, so the allocation-free call runs the best plan that fits;
    both stay within the oracle's tolerance on sampled columns."""
    layout, m, n, k = 0, 8192, 17408, 5120
    rng = np.random.default_rng(15100)
    w = synth.weights(rng, layout, n, k)
    a = synth.activations(rng, m, k, "bf16")
    wd, ad = torch.from_numpy(w).to(DEV), a.to(DEV).contiguous()
    c = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    st = noalloc(wd, layout, n, k, ad, c)
    assert st == R.RFP4_OK, R.rfp4_status_string(st)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([rng.choice(n, 24, replace=False), [0, n - 1025, n - 1024, n - 1]]))
    c_ref, den = O.gemm_rows(w, layout, n, k, a.to(torch.float64).numpy(), cols)
    assert gemm_error(c[:, cols].to(torch.float64).cpu().numpy(), c_ref, den) <= TOL


def test_noalloc_rejects_a_forced_plan_beyond_the_scratch():
    """Main tiles split four ways at 2048 x 17408 x 5120 need 544 MiB of partial sums:
    RFP4_ERR_SCRATCH, and nothing is launched (the output keeps its contents)."""
    layout, m, n, k = 0, 2048, 17408, 5120
    wd = torch.zeros((n, R.rfp4_row_bytes(layout, k)), dtype=torch.uint8, device=DEV)
    ad = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
    c = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=DEV)
    assert noalloc(wd, layout, n, k, ad, c, dict(gemm_plan="msplit4")) == R.RFP4_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((c == 7.0).all())
