"""GPU run-to-run determinism: repeated calls on the same inputs give bit-identical outputs,
on the calling stream and on a second stream (which gets its own split-tile workspace).

Every path sums in a fixed order: wavefront reductions, partial tiles met in a fixed
order by the last workgroup to arrive, split-k partials reduced by a separate kernel.
Atomics only count arrivals; no value is summed with them, so outputs may not depend on
scheduling. Inputs are drawn on the device from the seeded generators in synth/ at the
decode and prefill shapes.
"""

import pytest
import torch

import gemm_rfp4_block_amd as R
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def same_bits(a, b):
    ia = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
    ib = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
    return bool(torch.equal(ia, ib))


def three_runs(fn):
    """fn(stream) -> output tensor; two calls on the current stream, one on a side stream."""
    out0 = fn(None).clone()
    out1 = fn(None).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out2 = fn(side).clone()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return out0, out1, out2


GEMV_CASES = [
    # layout, n, k, batch, dtype, forced split of the matrix-core tiles (None = default)
    (0, 17408, 5120, 1, "f16", None),   # up-projection, dot-product kernel
    (1, 5120, 17408, 1, "bf16", None),  # down-projection, long rows
    (1, 5120, 17408, 2, "bf16", None),
    (1, 5120, 17408, 8, "bf16", None),
    (1, 5120, 17408, 4, "bf16", "4"),   # split tiles: partial sums + arrival counters
    (0, 6144, 5120, 3, "f16", "2"),
]


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "L{}n{}k{}b{}{}-s{}".format(*c))
def test_gemv_repeatable(case, force):
    layout, n, k, batch, dt, split = case
    if split is not None:
        force(gemv_splits=int(split))
    w = synth.weights_device(layout, n, k, 11, DEV)
    x = synth.activations_device(batch, k, dt, 12, DEV)
    outs = three_runs(lambda s: R.rfp4_gemv(w, layout, n, k, x, stream=s))
    assert torch.isfinite(outs[0]).all()
    assert same_bits(outs[0], outs[1]) and same_bits(outs[0], outs[2])


@pytest.mark.parametrize("ns,k", [([17408, 17408], 5120), ([6144, 1024, 1024], 5120)], ids=["gate_up", "qkv"])
def test_gemv_multi_repeatable(ns, k):
    ws = [synth.weights_device(0, n, k, 20 + i, DEV) for i, n in enumerate(ns)]
    x = synth.activations_device(1, k, "f16", 21, DEV)
    outs = three_runs(lambda s: torch.cat(R.rfp4_gemv_multi(ws, 0, ns, k, x, stream=s), dim=1))
    assert same_bits(outs[0], outs[1]) and same_bits(outs[0], outs[2])


GEMM_CASES = [
    # layout, m, n, k, forced plan ("" = the planner's choice)
    (0, 512, 17408, 5120, ""),
    (1, 256, 5120, 17408, ""),
    (0, 257, 520, 2304, "msplit3"),
    (0, 257, 520, 2304, "tail2"),
    (1, 100, 200, 512, "tail4"),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "L{}m{}n{}k{}-{}".format(*c))
def test_gemm_repeatable(case, force):
    layout, m, n, k, plan = case
    force(gemm_plan=plan or "auto")
    w = synth.weights_device(layout, n, k, 31, DEV)
    a = synth.activations_device(m, k, "bf16", 32, DEV)
    outs = three_runs(lambda s: R.rfp4_gemm(w, layout, n, k, a, stream=s))
    assert torch.isfinite(outs[0].float()).all()
    assert same_bits(outs[0], outs[1]) and same_bits(outs[0], outs[2])
