"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Acceptance: dequantization bit-exact (uint32 views, signs of zero included); GEMV and
GEMM max |y - y_ref| / sum |w x| <= 2e-3 (outputs with a zero denominator must be
exactly zero). Inputs come from the seeded generators in synth/. Full-size workloads
run in the launch configuration the benchmark times; the GEMM at full size is checked
on a seeded sample of output columns that the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

import gemm_rfp4_block_amd as R
import oracle.rfp4_oracle as O
import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x64(t):
    return t.to(torch.float64).cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def run_gemv(w, layout, n, k, x, ldx=None, ldy=None):
    """Call rfp4_gemv (through the binding, so the `force` fixture applies) with optional
    padded leading dimensions; returns (batch, n) fp32."""
    batch = x.shape[0]
    if ldx is None or ldx == k:
        xd = x.to(DEV).contiguous()
        ldx = k
    else:
        buf = torch.zeros((batch, ldx), dtype=x.dtype, device=DEV)
        buf[:, :k] = x.to(DEV)
        xd = buf
    ldy = n if ldy is None else ldy
    y = torch.full((batch, ldy), float("nan"), dtype=torch.float32, device=DEV)
    R.rfp4_gemv(dev(w), layout, n, k, xd, y)  # leading dimensions from the strides
    torch.cuda.synchronize()
    out = y.cpu().numpy()
    if ldy > n:
        assert np.all(np.isnan(out[:, n:])), "gemv wrote past n"
    return out[:, :n]


# ------------------------------------------------------------------ dequant

def test_dequant_tiny_bitwise():
    w, _, cfg = synth.gemv_inputs("tiny")
    n, k = cfg["n"], cfg["k"]
    got = R.rfp4_dequant(dev(w), cfg["layout"], n, k).cpu().numpy()
    assert np.array_equal(bits(got), bits(O.dequantize_f32(w, cfg["layout"], n, k)))


@pytest.mark.parametrize("layout", [0, 1])
def test_dequant_every_scale_byte_and_index(layout):
    """256 rows: row b uses scale byte b (dual: second half (b*37+11) % 256) on blocks
    that hold every one of the 16 indices in both nibble positions."""
    k = 512
    nb = k // 32
    qs = np.array([t | ((15 - t) << 4) for t in range(16)], dtype=np.uint8)
    rows = []
    for b in range(256):
        blk = []
        for j in range(nb):
            q = np.roll(qs, j)
            if layout == 0:
                blk.append(np.concatenate([q, [b, (b * 37 + 11) % 256]]).astype(np.uint8))
            else:
                blk.append(np.concatenate([q, [b]]).astype(np.uint8))
        rows.append(np.concatenate(blk))
    w = np.stack(rows)
    got = R.rfp4_dequant(dev(w), layout, 256, k).cpu().numpy()
    exp = O.dequantize_f32(w, layout, 256, k)
    assert np.array_equal(bits(got), bits(exp))


@pytest.mark.parametrize("name", ["up", "down"])
def test_dequant_full_size_bitwise(name):
    w, _, cfg = synth.gemv_inputs(name)
    n, k = cfg["n"], cfg["k"]
    got = R.rfp4_dequant(dev(w), cfg["layout"], n, k).cpu().numpy()
    exp = O.dequantize_f32(w, cfg["layout"], n, k)
    assert np.array_equal(bits(got), bits(exp))


def test_dequant_padded_ldo():
    rng = np.random.default_rng(21)
    n, k, ldo = 19, 512, 532
    w = synth.weights(rng, 1, n, k)
    out = torch.full((n, ldo), -7.0, dtype=torch.float32, device=DEV)
    R.rfp4_dequant(dev(w), 1, n, k, out=out, ldo=ldo)
    o = out.cpu().numpy()
    assert np.array_equal(bits(o[:, :k]), bits(O.dequantize_f32(w, 1, n, k)))
    assert np.all(o[:, k:] == -7.0)


def bf16_bits_of(f32):
    """bf16 encodings of fp32 values that are bf16 values (asserted: low 16 bits zero)."""
    u = bits(f32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def dequant_bf16_bits(w, layout, n, k, out=None):
    o = R.rfp4_dequant_bf16(dev(w), layout, n, k, out=out)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("layout", [0, 1])
def test_dequant_bf16_every_scale_byte_and_index(layout):
    """As the fp32 test: every scale byte, every index in both nibble positions, bf16
    output compared bit for bit (signs of zero included)."""
    k = 512
    nb = k // 32
    qs = np.array([t | ((15 - t) << 4) for t in range(16)], dtype=np.uint8)
    rows = []
    for b in range(256):
        blk = []
        for j in range(nb):
            q = np.roll(qs, 3 * j)
            sc = [b, (b * 37 + 11) % 256] if layout == 0 else [b]
            blk.append(np.concatenate([q, sc]).astype(np.uint8))
        rows.append(np.concatenate(blk))
    w = np.stack(rows)
    got = dequant_bf16_bits(w, layout, 256, k)
    assert np.array_equal(got, bf16_bits_of(O.dequantize_f32(w, layout, 256, k)))


@pytest.mark.parametrize("name", ["up", "down"])
def test_dequant_bf16_full_size_bitwise(name):
    w, _, cfg = synth.gemv_inputs(name)
    n, k = cfg["n"], cfg["k"]
    got = dequant_bf16_bits(w, cfg["layout"], n, k)
    assert np.array_equal(got, bf16_bits_of(O.dequantize_f32(w, cfg["layout"], n, k)))


def test_dequant_bf16_padded_ldo():
    rng = np.random.default_rng(22)
    n, k, ldo = 21, 1024, 1048
    w = synth.weights(rng, 0, n, k, stress_frac=0.05)
    out = torch.full((n, ldo), -3.0, dtype=torch.bfloat16, device=DEV)
    got = R.rfp4_dequant_bf16(dev(w), 0, n, k, out=out[:, :k])
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o[:, :k], bf16_bits_of(O.dequantize_f32(w, 0, n, k)))
    assert np.all(out[:, k:].float().cpu().numpy() == -3.0)
    assert got.data_ptr() == out.data_ptr()


# ------------------------------------------------------------------ GEMV

def check_gemv(w, layout, n, k, x, **kw):
    y = run_gemv(w, layout, n, k, x, **kw)
    y_ref, den = O.gemv(w, layout, n, k, x64(x))
    err = O.normalized_error(y, y_ref, den)
    assert err <= TOL, err
    return y, err


def test_gemv_tiny():
    w, x, cfg = synth.gemv_inputs("tiny")
    check_gemv(w, cfg["layout"], cfg["n"], cfg["k"], x)


def test_gemv_up_full():
    w, x, cfg = synth.gemv_inputs("up")
    check_gemv(w, cfg["layout"], cfg["n"], cfg["k"], x)


@pytest.mark.parametrize("batch", [2, 4, 8])
def test_gemv_up_full_batched(batch):
    """The up-projection weights at batches 2/4/8 on the default path (the matrix-core
    tile kernel: one tile per workgroup, unsplit), every output against the oracle."""
    w, _, cfg = synth.gemv_inputs("up")
    x = synth.activations(np.random.default_rng(9900 + batch), batch, cfg["k"], cfg["xdtype"])
    check_gemv(w, cfg["layout"], cfg["n"], cfg["k"], x)


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_gemv_down_full_stress(batch):
    w, x, cfg = synth.gemv_inputs("down", batch=batch)
    check_gemv(w, cfg["layout"], cfg["n"], cfg["k"], x)


RAGGED = [  # layout, n, k, batch, dtype, ldx, ldy
    (0, 1, 256, 1, "f16", None, None),
    (0, 3, 768, 2, "bf16", 776, 9),
    (0, 37, 2304, 3, "f16", None, 40),
    (0, 130, 256, 8, "bf16", 264, None),
    (0, 257, 4096, 5, "f16", None, None),
    (1, 1, 512, 1, "bf16", None, None),
    (1, 45, 1536, 6, "f16", 1544, 48),
    (1, 67, 512, 7, "bf16", None, None),
    (1, 300, 8192, 8, "f16", None, None),
    (0, 1000, 6144, 1, "bf16", None, None),
    (1, 513, 17408, 1, "f16", None, None),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "L{}n{}k{}b{}{}".format(*c[:5]))
def test_gemv_ragged(case):
    layout, n, k, batch, dt, ldx, ldy = case
    rng = np.random.default_rng(1000 + n + k + batch)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, batch, k, dt)
    check_gemv(w, layout, n, k, x, ldx=ldx, ldy=ldy)


# Forced lane mappings "P:CL": P blocks per lane unit, CL lanes per row. Cases where CL
# does not divide the units of a row exercise the masked remainder; the activations are
# staged in LDS for the small shapes and read from global memory for the long rows.
GEMV_PLANS = [
    ("1:64", 0, 75, 2304, 1, "f16"), ("2:64", 0, 75, 2304, 3, "bf16"), ("2:32", 1, 33, 1536, 2, "f16"),
    ("1:16", 1, 19, 1536, 1, "bf16"), ("2:8", 0, 130, 768, 8, "f16"), ("1:64", 1, 40, 17408, 1, "bf16"),
    ("2:64", 1, 40, 17408, 2, "bf16"), ("1:32", 0, 9, 256, 1, "f16"),
]


@pytest.mark.parametrize("case", GEMV_PLANS, ids=lambda c: "{}-L{}n{}k{}b{}{}".format(*c))
def test_gemv_forced_plan(case, force):
    plan, layout, n, k, batch, dt = case
    force(gemv_kernel="dot", gemv_plan=tuple(map(int, plan.split(":"))))  # dot-product lane mappings
    rng = np.random.default_rng(5000 + n + k + batch)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, batch, k, dt)
    check_gemv(w, layout, n, k, x, ldy=n + 3)


# Tall launches with few lanes per row, so that a wavefront walks two row groups: the
# busiest lanes then hold more units than one round of loads (depth 2), and lanes with
# one group fewer end on a round that repeats loads (the launch's first unit, never
# consumed). Both layouts, both kinds of unit (pairs of 36 / 34 bytes, single blocks
# realigned from word boundaries), batch 1 and 2.
ROUNDS = [  # plan, layout, n, k, batch, dtype
    ("1:8", 0, 65536, 768, 1, "f16"), ("1:8", 1, 65536, 768, 1, "bf16"),
    ("2:8", 1, 65536, 768, 2, "f16"), ("2:8", 0, 65536, 1536, 2, "bf16"),
    ("2:4", 1, 30000, 2304, 1, "bf16"),
]


@pytest.mark.parametrize("case", ROUNDS, ids=lambda c: "{}-L{}n{}k{}b{}{}".format(*c))
def test_gemv_rounds_over_several_row_groups(case, force):
    plan, layout, n, k, batch, dt = case
    force(gemv_kernel="dot", gemv_plan=tuple(map(int, plan.split(":"))))
    rng = np.random.default_rng(5500 + n + k + batch)
    w = synth.weights(rng, layout, n, k, stress_frac=0.01)
    x = synth.activations(rng, batch, k, dt)
    check_gemv(w, layout, n, k, x, ldy=n + 1)


MULTI = [  # layout, [n per part], k, batch, dtype
    (0, [17408, 17408], 5120, 1, "f16"),       # gate + up
    (0, [6144, 1024, 1024], 5120, 1, "f16"),   # q, k, v
    (1, [300, 45, 1000, 7], 1536, 3, "bf16"),
    (0, [1, 2, 3, 4, 5, 6, 7, 8], 256, 8, "f16"),
    (1, [513, 64], 17408, 2, "bf16"),
]


@pytest.mark.parametrize("case", MULTI, ids=lambda c: "L{}p{}k{}b{}{}".format(c[0], len(c[1]), *c[2:]))
def test_gemv_multi(case):
    layout, ns, k, batch, dt = case
    rng = np.random.default_rng(6000 + sum(ns) + k + batch)
    ws = [synth.weights(rng, layout, n, k, stress_frac=0.01) for n in ns]
    x = synth.activations(rng, batch, k, dt)
    xd = x.to(DEV).contiguous()
    ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, ns, k, xd)
    torch.cuda.synchronize()
    for w, n, y in zip(ws, ns, ys):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


def test_gemv_multi_equals_single_calls(force):
    """With the same (forced) lane mapping the fused launch gives exactly the results of
    separate calls."""
    force(gemv_kernel="dot", gemv_plan=(2, 16))
    rng = np.random.default_rng(77)
    ns, k = [640, 96, 96], 2048
    ws = [dev(synth.weights(rng, 0, n, k)) for n in ns]
    xd = synth.activations(rng, 2, k, "f16").to(DEV).contiguous()
    ys = R.rfp4_gemv_multi(ws, 0, ns, k, xd)
    singles = [R.rfp4_gemv(w, 0, n, k, xd) for w, n in zip(ws, ns)]
    torch.cuda.synchronize()
    for y, s1 in zip(ys, singles):
        assert torch.equal(y, s1)


NONFINITE_X = [  # kernel, plan, layout, n, k, batch, dtype
    ("0", "2:32", 1, 40, 17408, 2, "bf16"),  # dot product, 272 units over 32 lanes: ragged
    ("0", "1:64", 0, 21, 4000, 1, "f16"),    # dot product, 125 single blocks over 64 lanes
    ("0", "1:64", 1, 40, 17408, 8, "bf16"),  # dot product, activations from global memory
    ("1", None, 0, 33, 1408, 3, "f16"),      # matrix cores, 22 units: last chunk 6 of 16
    ("1", None, 1, 45, 1056, 8, "bf16"),     # matrix cores, 33 single blocks
]


@pytest.mark.parametrize("case", NONFINITE_X, ids=lambda c: "mfma{}-{}-L{}n{}k{}b{}{}".format(*c))
def test_gemv_nonfinite_activations(case, force):
    """An infinite activation in the last block of a row: rows whose exact sum is +-inf
    (or NaN, where a zero weight meets it) give exactly that; lanes or lane groups past
    the row end, which re-read that last block, must add nothing (not 0 * inf = NaN).
    Other activation rows stay finite and within tolerance."""
    mode, plan, layout, n, k, batch, dt = case
    force(gemv_kernel={"0": "dot", "1": "tiles"}[mode],
          gemv_plan=tuple(map(int, plan.split(":"))) if plan is not None else None)
    rng = np.random.default_rng(9300 + n + k)
    w = synth.weights(rng, layout, n, k)
    x = synth.activations(rng, batch, k, dt)
    x[0, k - 1] = float("inf")
    if batch > 2:
        x[2, k - 33] = float("-inf")
    y = R.rfp4_gemv(dev(w), layout, n, k, x.to(DEV).contiguous()).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):  # 0 * inf in the exact sums
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
    nonfinite = ~np.isfinite(y_ref)
    assert nonfinite[0].all()
    assert np.array_equal(np.isnan(y), np.isnan(y_ref))
    assert np.array_equal(y[nonfinite & ~np.isnan(y_ref)], y_ref[nonfinite & ~np.isnan(y_ref)])
    rows = np.isfinite(y_ref).all(axis=1)
    if rows.any():
        assert O.normalized_error(y[rows], y_ref[rows], den[rows]) <= TOL


TALL_CASES = [  # row counts of the matrices (one launch), k, activation dtype, layout
    ([48], 5120, "f16", 0),             # three tiles
    ([16], 6144, "f16", 0),             # one tile, six units per lane
    ([160], 5120, "f16", 0),
    ([32, 48, 16], 5120, "f16", 0),     # fused parts (tiles map to matrices)
    ([64, 16], 6144, "f16", 0),
    ([40], 5120, "f16", 0),             # rows not a multiple of 16: dot-product kernel
    ([48], 4096, "f16", 0),             # k outside {5120, 6144}: dot-product kernel
    ([48], 5120, "f16", 1),             # fast layout: dot-product kernel
    ([48], 5120, "bf16", 0),            # bf16 activations: dot-product kernel
]


@pytest.mark.parametrize("case", TALL_CASES, ids=lambda c: "n{}k{}{}L{}".format("-".join(map(str, c[0])), *c[1:]))
def test_gemv_tall_forced(case, force):
    """The batch-1 matrix-core kernel for tall launches, forced on wherever the shape
    allows (the tall kernel forced through rfp4_force), against the oracle; shapes it does not take fall back to
    the dot-product kernel and must stay correct. Weights include 2 % stress blocks
    (extreme codes and scales)."""
    force(gemv_kernel="tall")
    ns, k, dt, layout = case
    rng = np.random.default_rng(9900 + sum(ns) + k + layout)
    ws = [synth.weights(rng, layout, n, k, stress_frac=0.02) for n in ns]
    x = synth.activations(rng, 1, k, dt)
    xd = x.to(DEV).contiguous()
    if len(ns) == 1:
        ys = [R.rfp4_gemv(dev(ws[0]), layout, ns[0], k, xd)]
    else:
        ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, ns, k, xd)
    for w, n, y in zip(ws, ns, ys):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


def test_gemv_tall_nonfinite_activations(force):
    """Tall kernel: an infinite activation in the last unit of the rows gives exactly the
    oracle's +-inf or NaN (a zero weight or a zero scale meeting it); the zero-padded A
    rows add nothing."""
    force(gemv_kernel="tall")
    layout, n, k = 0, 64, 5120
    rng = np.random.default_rng(9950)
    w = synth.weights(rng, layout, n, k, stress_frac=0.05)
    x = synth.activations(rng, 1, k, "f16")
    x[0, k - 1] = float("inf")
    x[0, k - 40] = float("-inf")
    y = R.rfp4_gemv(dev(w), layout, n, k, x.to(DEV).contiguous()).cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
    assert np.array_equal(np.isnan(y), np.isnan(y_ref))
    inf = np.isinf(y_ref)
    assert np.array_equal(y[inf], y_ref[inf])
    fin = np.isfinite(y_ref)
    if fin.any():
        assert np.max(np.abs(y[fin] - y_ref[fin]) / den[fin]) <= TOL


def test_gemv_tall_default_fused_qkv():
    """By default a fused q + k + v launch (6144 + 1024 + 1024 rows x 5120, dual, f16,
    batch 1: two 16-row tiles per CU) takes the tall kernel; every row of every part
    against the oracle."""
    layout, k, ns = 0, 5120, [6144, 1024, 1024]
    rng = np.random.default_rng(9970)
    ws = [synth.weights(rng, layout, n, k, stress_frac=0.01) for n in ns]
    x = synth.activations(rng, 1, k, "f16")
    ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, ns, k, x.to(DEV).contiguous())
    for w, n, y in zip(ws, ns, ys):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


def test_gemv_tall_default_fused_gate_up_sampled():
    """By default a fused gate + up launch (2 x 17408 x 5120, dual, f16, batch 1: >= 8
    tiles per CU) takes the tall kernel; checked on seeded sampled rows of both matrices
    (first and last rows included)."""
    layout, n, k = 0, 17408, 5120
    rng = np.random.default_rng(9960)
    ws = [synth.weights(rng, layout, n, k) for _ in range(2)]
    x = synth.activations(rng, 1, k, "f16")
    ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, [n, n], k, x.to(DEV).contiguous())
    for w, y in zip(ws, ys):
        rows = np.unique(np.concatenate([[0, 1, 15, 16, n - 17, n - 16, n - 1], rng.choice(n, 64, replace=False)]))
        y_ref, den = O.gemv_rows(w, layout, n, k, x64(x), rows)
        assert O.normalized_error(y.cpu().numpy()[:, rows], y_ref, den) <= TOL


@pytest.mark.parametrize("n,kernel", [(32768, "auto"), (33792, "tall")])
def test_gemv_tall_staged_sampled(n, kernel, force):
    """From 8 tiles per CU the tall kernel loads its weights along rows and hands them to
    the multiplying lanes through a double-buffered LDS stage: a single 32768-row matrix
    takes it by default, and 33792 rows (tiles spread unevenly over the CUs) when forced.
    Weights include 2 % stress blocks; seeded sampled rows (both ends of the matrix and
    of tiles included) against the oracle, and every row against the dot-product kernel."""
    layout, k = 0, 5120
    rng = np.random.default_rng(9970 + n)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, 1, k, "f16")
    wd, xd = dev(w), x.to(DEV).contiguous()
    force(gemv_kernel=kernel)
    y = R.rfp4_gemv(wd, layout, n, k, xd).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 4095, 4096, n - 17, n - 16, n - 1],
                                     rng.choice(n, 96, replace=False)]))
    y_ref, den = O.gemv_rows(w, layout, n, k, x64(x), rows)
    assert O.normalized_error(y[:, rows], y_ref, den) <= TOL
    force(gemv_kernel="dot")
    y_dot = R.rfp4_gemv(wd, layout, n, k, xd).cpu().numpy()
    assert np.all(np.isfinite(y)) and np.allclose(y, y_dot, rtol=2e-3, atol=1e-3 * np.abs(y_dot).max())


def test_gemv_zero_scales_give_zero():
    rng = np.random.default_rng(31)
    n, k = 64, 1024
    w = synth.weights(rng, 0, n, k).reshape(n, k // 32, 18)
    w[:, :, 16:] = np.where(rng.integers(0, 2, size=w[:, :, 16:].shape) == 1, 0x80, 0x00)
    x = synth.activations(rng, 3, k, "f16")
    y = run_gemv(w.reshape(n, -1), 0, n, k, x)
    assert np.all(y == 0.0)


def test_gemv_one_hot_selects_a_column():
    rng = np.random.default_rng(32)
    n, k = 96, 2048
    w = synth.weights(rng, 0, n, k)
    wd = O.dequantize_f32(w, 0, n, k)
    for j in (0, 31, 32, 1000, 2047):
        x = torch.zeros((1, k), dtype=torch.float16)
        x[0, j] = 1.0
        y = run_gemv(w, 0, n, k, x)
        assert np.array_equal(y[0], wd[:, j])  # numeric equality: one exact product


def test_gemv_extreme_values():
    """Largest finite scales, all-magnitude-10 codes and the largest fp16 activations:
    the fp32 accumulation must neither overflow nor lose the result."""
    n, k = 16, 4096
    rng = np.random.default_rng(33)
    w = synth.weights(rng, 0, n, k).reshape(n, k // 32, 18)
    w[:, :, :16] = np.where(rng.integers(0, 2, size=(n, k // 32, 16)) == 1, 0xF7, 0x7F)
    w[:, :, 16:] = 0x7E
    x = torch.full((2, k), 65504.0, dtype=torch.float16)
    x[1, ::2] = -65504.0
    check_gemv(w.reshape(n, -1), 0, n, k, x)


@pytest.mark.parametrize("layout,dt", [(0, "f16"), (1, "bf16")])
def test_gemv_exact_invariants(layout, dt):
    """The default batch-4 launch (the tile kernel): +1 on every scale exponent field
    doubles y bitwise (the scale enters through exact operations); two runs agree
    bitwise (fixed reduction order, no atomics). Toggling every index sign negates y to
    within rounding: the matrix cores' fp32 accumulation is not sign-symmetric in every
    case (measured on gfx950, see test_gpu_scale_range.py), so an exactly negated input
    can come back an fp32 ulp or two away from the negated output."""
    rng = np.random.default_rng(34 + layout)
    n, k = 200, 4096
    w = synth.weights(rng, layout, n, k)
    x = synth.activations(rng, 4, k, dt)
    bb = synth.block_bytes(layout)
    y = run_gemv(w, layout, n, k, x)
    y_again = run_gemv(w, layout, n, k, x)
    assert np.array_equal(bits(y), bits(y_again))
    blocks = w.reshape(n, k // 32, bb)
    flip = blocks.copy()
    flip[:, :, :16] ^= 0x88
    yf = run_gemv(flip.reshape(n, -1), layout, n, k, x)
    _, den = O.gemv(w, layout, n, k, x64(x))
    assert np.all(np.abs(yf.astype(np.float64) + y) <= 2.0 ** -20 * den)
    step = blocks.copy()
    step[:, :, 16:] += 8
    ys = run_gemv(step.reshape(n, -1), layout, n, k, x)
    assert np.array_equal(ys, 2 * y)


def test_gemv_dual_equal_halves_matches_fast():
    rng = np.random.default_rng(36)
    n, k = 128, 2048
    wf = synth.weights(rng, 1, n, k).reshape(n, k // 32, 17)
    wd = np.concatenate([wf, wf[:, :, 16:]], axis=2)
    x = synth.activations(rng, 2, k, "bf16")
    yf = run_gemv(wf.reshape(n, -1), 1, n, k, x)
    yd = run_gemv(wd.reshape(n, -1), 0, n, k, x)
    assert np.array_equal(bits(yf), bits(yd))


# ------------------------------------------------------------------ GEMM

def gemm_error(c, c_ref, den):
    """Normalized error of a bf16-output GEMM. The output format adds its own rounding
    (half a bf16 ulp of the exact value, up to 2^-8 relative), which the page does not
    budget for; that part is allowed on top of the 2e-3 bound, which applies to the rest."""
    c = np.asarray(c, dtype=np.float64)
    mag = np.abs(c_ref)
    half_ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 8), 0.0)
    excess = np.maximum(np.abs(c - c_ref) - half_ulp, 0.0)
    return O.normalized_error(c_ref + np.sign(c - c_ref) * excess, c_ref, den)


def run_gemm(w, layout, n, k, a, ldc=None):
    m = a.shape[0]
    ad = a.to(DEV).contiguous()
    ldc = n if ldc is None else ldc
    c = torch.full((m, ldc), float("nan"), dtype=torch.bfloat16, device=DEV)
    R.rfp4_gemm(dev(w), layout, n, k, ad, c)  # ldc from the stride; the force fixture applies
    torch.cuda.synchronize()
    out = c.to(torch.float64).cpu().numpy()
    if ldc > n:
        assert np.all(np.isnan(out[:, n:])), "gemm wrote past n"
    return out[:, :n]


GEMM_CASES = [  # layout, m, n, k
    (0, 1, 1, 256), (0, 100, 200, 512), (1, 77, 129, 1024), (0, 128, 128, 256),
    (0, 257, 300, 2304), (1, 33, 513, 512), (0, 512, 64, 5120),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "L{}m{}n{}k{}".format(*c))
def test_gemm_small(case):
    layout, m, n, k = case
    rng = np.random.default_rng(2000 + m + n + k)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    a = synth.activations(rng, m, k, "bf16")
    ldc = (n + 7) // 8 * 8 + 8  # padded leading dimension, multiple of 8
    c = run_gemm(w, layout, n, k, a, ldc=ldc)
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c, c_ref, den) <= TOL


@pytest.mark.parametrize("case", [(0, 100, 200, 512), (1, 77, 136, 1024), (0, 1, 8, 256), (0, 257, 296, 2304)])
def test_gemm_ragged_mn(case):
    layout, m, n, k = case
    rng = np.random.default_rng(3000 + m + n)
    w = synth.weights(rng, layout, n, k)
    a = synth.activations(rng, m, k, "bf16")
    c = run_gemm(w, layout, n, k, a)
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c, c_ref, den) <= TOL


def test_gemm_same_sign_rounding():
    """All terms positive: the bf16 output must be within one bf16 ulp of the exactly
    rounded oracle value (the normalized metric alone would be dominated by rounding)."""
    m, n, k = 64, 64, 1024
    rng = np.random.default_rng(41)
    w = synth.weights(rng, 0, n, k).reshape(n, k // 32, 18)
    w[:, :, :16] &= 0x77  # clear both sign bits: all codes >= 0
    w = w.reshape(n, -1)
    a = torch.from_numpy(np.abs(rng.standard_normal((m, k))).astype(np.float32)).to(torch.bfloat16)
    c = run_gemm(w, 0, n, k, a)
    c_ref, _ = O.gemm(w, 0, n, k, x64(a))
    ref_bf = torch.from_numpy(c_ref).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    ulp = np.abs(ref_bf) * 2.0 ** -7
    assert np.all(np.abs(c - ref_bf) <= ulp + 1e-30)


@pytest.mark.parametrize("plan", ["main", "tail", "tail2", "tail4", "msplit2", "msplit3", "msplit4"])
@pytest.mark.parametrize("case", [(0, 100, 200, 512), (1, 77, 136, 1024), (0, 257, 520, 2304),
                                  (1, 300, 264, 512)], ids=lambda c: "L{}m{}n{}k{}".format(*c))
def test_gemm_forced_tile_size(case, plan, force):
    """Each tile configuration alone over the whole matrix, ragged edges included."""
    force(gemm_plan=plan)
    layout, m, n, k = case
    rng = np.random.default_rng(4000 + m + n + k)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    a = synth.activations(rng, m, k, "bf16")
    c = run_gemm(w, layout, n, k, a, ldc=n + 8)
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c, c_ref, den) <= TOL


def test_gemm_split_main_tiles_full_size_sampled(force):
    """The 2048 x 5120 x 17408 down-projection prefill, for which the planner splits the
    k range of the 256 x 256 tiles three ways; checked on sampled columns."""
    layout, m, n, k = 1, 2048, 5120, 17408
    w = synth.weights(np.random.default_rng(4400), layout, n, k, stress_frac=0.01)
    a = synth.activations(np.random.default_rng(4401), m, k, "bf16")
    c = run_gemm(w, layout, n, k, a)
    cols = np.unique(np.concatenate([np.random.default_rng(4402).choice(n, 40, replace=False), [0, 255, 256, n - 1]]))
    c_ref, den = O.gemm_rows(w, layout, n, k, x64(a), cols)
    assert gemm_error(c[:, cols], c_ref, den) <= TOL


def test_gemm_large_ragged_m_sampled():
    """3000 token rows (not a multiple of the 256-row tile) against the 17408 x 5120
    up-projection: more than four rounds of main tiles plus the planner's tail; sampled
    columns, every row, including the last partial row tile."""
    layout, m, n, k = 0, 3000, 17408, 5120
    w = synth.weights(np.random.default_rng(4500), layout, n, k)
    a = synth.activations(np.random.default_rng(4501), m, k, "bf16")
    c = run_gemm(w, layout, n, k, a)
    edges = np.array([0, 255, 256, n - 1025, n - 1024, n - 257, n - 256, n - 1])
    cols = np.unique(np.concatenate([np.random.default_rng(4502).choice(n, 40, replace=False), edges]))
    c_ref, den = O.gemm_rows(w, layout, n, k, x64(a), cols)
    assert gemm_error(c[:, cols], c_ref, den) <= TOL
    assert np.all(np.isfinite(c))


def test_gemm_mixed_tile_sizes():
    """2048 x 8448: 256 full tiles plus one strip of 256 columns that the launcher computes
    as 128 x 128 tiles with the k range split in two (partial sums, then a reduction);
    every output is compared, across the boundary at column 8192."""
    layout, m, n, k = 0, 2048, 8448, 256
    rng = np.random.default_rng(4321)
    w = synth.weights(rng, layout, n, k, stress_frac=0.01)
    a = synth.activations(rng, m, k, "bf16")
    c = run_gemm(w, layout, n, k, a)
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c, c_ref, den) <= TOL


@pytest.mark.parametrize("case", [(0, 100, 200, 512), (1, 77, 136, 1024), (0, 257, 520, 2304)],
                         ids=lambda c: "L{}m{}n{}k{}".format(*c))
def test_gemm_dequant_fallback(case):
    """Dequantize to bf16 + dense GEMM: same tolerance as the fused GEMM; the bf16
    weight buffer holds the exact dequantization afterwards."""
    layout, m, n, k = case
    rng = np.random.default_rng(7000 + m + n + k)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    a = synth.activations(rng, m, k, "bf16")
    wbuf = torch.empty((n, k), dtype=torch.bfloat16, device=DEV)
    c = R.rfp4_gemm_dequant(dev(w), layout, n, k, a.to(DEV).contiguous(), wbuf=wbuf)
    torch.cuda.synchronize()
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c.to(torch.float64).cpu().numpy(), c_ref, den) <= TOL
    wb = wbuf.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(wb, bf16_bits_of(O.dequantize_f32(w, layout, n, k)))


def test_gemm_dequant_full_size_sampled():
    w, a, cfg = synth.gemm_inputs("prefill")
    n, k, m = cfg["n"], cfg["k"], cfg["m"]
    c = R.rfp4_gemm_dequant(dev(w), cfg["layout"], n, k, a.to(DEV).contiguous())
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(98).choice(n, size=64, replace=False))
    c_ref, den = O.gemm_rows(w, cfg["layout"], n, k, x64(a), cols)
    assert gemm_error(c[:, cols].to(torch.float64).cpu().numpy(), c_ref, den) <= TOL


XCD_GRID_CASES = [  # m, n, k, and the XCD grid (M groups) the launcher's byte model picks
    (256, 4096, 1024, 1),    # one M tile: the XCDs split the N strips only
    (1024, 4096, 2048, 2),
    (2048, 2048, 4096, 4),
    (4096, 2048, 1024, 8),   # A much larger than W: the XCDs split the M tiles only
]


@pytest.mark.parametrize("case", XCD_GRID_CASES, ids=lambda c: "m{}n{}k{}-mg{}".format(*c))
def test_gemm_xcd_tile_grid(case, force):
    """Main tiles only, on shapes whose tile counts give each of the XCD grids of the tile
    order (M groups 1, 2, 4, 8): every output is written (the order is a bijection of the
    tiles; C starts as NaN) and sampled columns, the first and last of each 256-column
    strip included, match the oracle."""
    m, n, k, _ = case
    force(gemm_plan="main")
    layout = 0
    w = synth.weights(np.random.default_rng(4600 + m + n), layout, n, k)
    a = synth.activations(np.random.default_rng(4601 + k), m, k, "bf16")
    c = run_gemm(w, layout, n, k, a)
    assert np.all(np.isfinite(c))
    rng = np.random.default_rng(4602)
    strips = np.arange(0, n, 256)
    cols = np.unique(np.concatenate([rng.choice(n, size=24, replace=False), strips, strips + 255]))
    c_ref, den = O.gemm_rows(w, layout, n, k, x64(a), cols)
    assert gemm_error(c[:, cols], c_ref, den) <= TOL


def test_gemm_full_size_sampled():
    w, a, cfg = synth.gemm_inputs("prefill")
    n, k, m = cfg["n"], cfg["k"], cfg["m"]
    c = run_gemm(w, cfg["layout"], n, k, a)
    rng = np.random.default_rng(99)
    # Random columns plus the edges of the last 256-column strips, where the launcher
    # may switch tile size.
    edges = np.array([0, 255, 256, n - 1025, n - 1024, n - 513, n - 512, n - 257, n - 256, n - 65, n - 64, n - 1])
    cols = np.unique(np.concatenate([rng.choice(n, size=96, replace=False), edges]))
    c_ref, den = O.gemm_rows(w, cfg["layout"], n, k, x64(a), cols)
    assert gemm_error(c[:, cols], c_ref, den) <= TOL
    assert np.all(np.isfinite(c))


# ------------------------------------------------------------------ quantize

QDT = {"f32": (torch.float32, R.RFP4_F32), "bf16": (torch.bfloat16, R.RFP4_BF16),
       "f16": (torch.float16, R.RFP4_F16)}


def run_quantize(src, layout, lds=None):
    """rfp4_quantize on a CPU tensor (n, k); columns k..lds-1 of a padded source hold
    NaN (a read past k would saturate its group). Returns uint8 (n, row_bytes)."""
    n, k = src.shape
    code = {torch.float32: R.RFP4_F32, torch.bfloat16: R.RFP4_BF16, torch.float16: R.RFP4_F16}[src.dtype]
    lds = k if lds is None else lds
    sd = torch.full((n, lds), float("nan"), dtype=src.dtype, device=DEV)
    sd[:, :k] = src.to(DEV)
    rb = synth.row_bytes(layout, k)
    out = torch.full((n * rb + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    st = R.lib().rfp4_quantize(R._ptr(sd), code, n, k, lds, layout, R._ptr(out), R._stream(None))
    assert st == R.RFP4_OK, R.rfp4_status_string(st)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[n * rb:] == 0xA5), "quantize wrote past its output"
    return o[: n * rb].reshape(n, rb)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("shape", [(37, 800), (1, 32), (5, 96), (300, 544)], ids=lambda s: "n{}k{}".format(*s))
def test_quantize_matches_oracle(shape, layout, dt):
    """Byte-exact against the oracle; (37, 800) spans several 256-block segments and
    ends on a partial one whose byte count is not a multiple of 16."""
    n, k = shape
    src = synth.real_weights(np.random.default_rng(n * 7 + k), n, k, dt)
    got = run_quantize(src, layout)
    assert np.array_equal(got, O.quantize(x64(src), layout))


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("layout", [0, 1])
def test_quantize_padded_rows(layout, dt):
    n, k, lds = 33, 256, 264
    src = synth.real_weights(np.random.default_rng(5), n, k, dt)
    assert np.array_equal(run_quantize(src, layout, lds), O.quantize(x64(src), layout))


def quantize_edge_rows(dt):
    """Rows of 128 values: zeros and negative zeros; NaN and infinities; saturation;
    exact ties at a normal and a subnormal scale; tiny values; mixed magnitudes."""
    big = {"f32": 3e38, "bf16": 3e38, "f16": 60000.0}[dt]
    tiny = {"f32": 1e-30, "bf16": 1e-30, "f16": 6e-8}[dt]
    rows = np.zeros((8, 128), dtype=np.float64)
    rows[0, 3] = -0.0
    rows[0, 40:48] = -0.0
    rows[1, 0] = np.nan
    rows[1, 5] = 1.0
    rows[1, 20] = np.inf
    rows[1, 40] = -np.inf
    rows[1, 41] = -3.0
    rows[1, 70] = np.nan
    rows[1, 71] = -np.inf
    rows[2, :32] = big
    rows[2, 32:64] = -big * np.linspace(0, 1, 32)
    ties = np.array([0.5, 1.5, 2.5, 3.5, 5.0, 7.0, 9.0, 10.0, 0.25, 4.0, 6.0, 8.0, 1.0, 2.0, 3.0, 9.5])
    s_norm = 0.5 * 1.375 * 2.0 ** -1   # decoded scale of byte 0x33
    s_sub = 5 * 2.0 ** -10              # decoded scale of byte 0x05
    rows[3] = np.concatenate([ties, -ties, ties[::-1], -ties[::-1]] * 2) * s_norm
    rows[4] = np.concatenate([ties, -ties, ties[::-1], -ties[::-1]] * 2) * s_sub
    rows[5] = tiny * np.arange(128) * (-1.0) ** np.arange(128)
    rows[6] = np.exp2(np.arange(128) % 30 - 15.0) * (-1.0) ** (np.arange(128) // 3)
    rows[7, ::16] = 2240.0  # 10 * S(126), the largest finite reach
    rows[7, 1::16] = 2240.0 * (1 + 2.0 ** -10)
    t = torch.from_numpy(rows).to(QDT[dt][0])
    return t


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("layout", [0, 1])
def test_quantize_edge_cases(layout, dt):
    src = quantize_edge_rows(dt)
    got = run_quantize(src, layout)
    ref = O.quantize(x64(src), layout)
    assert np.array_equal(got, ref)
    sb = got.reshape(8, 4, synth.block_bytes(layout))[:, :, 16:]
    assert np.all(sb <= 126)
    assert np.all(got[0] == 0)


@pytest.mark.parametrize("layout,dt", [(0, "bf16"), (1, "f32"), (0, "f16")])
def test_quantize_full_size_sampled(layout, dt):
    """The up-projection shape (17408 x 5120) in one launch; rows are independent, so
    the oracle checks a seeded sample of rows plus the first and last."""
    n, k = 17408, 5120
    src = synth.real_weights(np.random.default_rng(3), n, k, dt)
    got = run_quantize(src, layout)
    rows = np.unique(np.concatenate([np.random.default_rng(4).choice(n, 48, replace=False), [0, n - 1]]))
    assert np.array_equal(got[rows], O.quantize(x64(src[rows]), layout))


# ------------------------------------------------------------------ rows of any length
# k % 32 == 0 only: row lengths that are not multiples of 16 bytes (so rows start at
# every byte offset), odd block counts (single-block GEMV units), block counts that are
# not multiples of four (the GEMM's zero-filled k tail) and one-block rows.

UNALIGNED_DQ = [(0, 37, 96), (1, 29, 96), (0, 5, 32), (1, 7, 32), (0, 33, 1408), (1, 31, 544),
                (1, 19, 1056), (0, 3, 4000)]


@pytest.mark.parametrize("case", UNALIGNED_DQ, ids=lambda c: "L{}n{}k{}".format(*c))
def test_unaligned_rows_dequant_bitwise(case):
    layout, n, k = case
    w = synth.weights(np.random.default_rng(8000 + n + k), layout, n, k, stress_frac=0.05)
    wd = dev(w)
    ref = O.dequantize_f32(w, layout, n, k)
    got = R.rfp4_dequant(wd, layout, n, k).cpu().numpy()
    assert np.array_equal(bits(got), bits(ref))
    out = torch.empty((n, (k + 7) // 8 * 8), dtype=torch.bfloat16, device=DEV)
    R.rfp4_dequant_bf16(wd, layout, n, k, out)
    torch.cuda.synchronize()
    gb = out[:, :k].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(gb, bf16_bits_of(ref))


UNALIGNED_GEMV = [  # layout, n, k, batch, dtype
    (0, 257, 96, 1, "f16"), (1, 255, 96, 3, "bf16"), (0, 100, 1408, 1, "bf16"), (1, 99, 1056, 8, "f16"),
    (1, 33, 32, 2, "bf16"), (0, 1, 32, 1, "f16"), (0, 300, 4000, 1, "bf16"), (1, 77, 4000, 2, "f16"),
    (1, 130, 1088, 4, "bf16"), (0, 64, 100000, 1, "f16"), (1, 40, 99968, 2, "bf16"),
]


@pytest.mark.parametrize("case", UNALIGNED_GEMV, ids=lambda c: "L{}n{}k{}b{}{}".format(*c))
def test_unaligned_rows_gemv(case):
    layout, n, k, batch, dt = case
    rng = np.random.default_rng(8100 + n + k + batch)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, batch, k, dt)
    check_gemv(w, layout, n, k, x, ldy=n + 1)


@pytest.mark.parametrize("plan", ["1:1", "1:4", "1:64", "2:2", "2:16"])
@pytest.mark.parametrize("case", [(0, 70, 1408, 2, "f16"), (1, 61, 1088, 1, "bf16"), (1, 45, 1056, 3, "f16")],
                         ids=lambda c: "L{}n{}k{}b{}{}".format(*c))
def test_unaligned_rows_gemv_forced_plan(case, plan, force):
    """Every lane mapping on rows at all byte offsets (an odd block count ignores a
    forced P = 2 and takes single-block units)."""
    force(gemv_kernel="dot", gemv_plan=tuple(map(int, plan.split(":"))))
    layout, n, k, batch, dt = case
    rng = np.random.default_rng(8200 + n + k)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, batch, k, dt)
    check_gemv(w, layout, n, k, x)


def test_unaligned_rows_gemv_multi():
    layout, ns, k, batch = 1, [33, 1, 70, 5], 1056, 2
    rng = np.random.default_rng(8300)
    ws = [synth.weights(rng, layout, n, k, stress_frac=0.01) for n in ns]
    x = synth.activations(rng, batch, k, "bf16")
    ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, ns, k, x.to(DEV).contiguous())
    torch.cuda.synchronize()
    for w, n, y in zip(ws, ns, ys):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


UNALIGNED_GEMM = [  # layout, m, n, k
    (0, 100, 200, 96), (1, 77, 136, 160), (0, 257, 520, 1408), (1, 64, 300, 1056), (0, 1, 8, 32),
    (1, 130, 129, 544), (0, 33, 64, 224),
]


@pytest.mark.parametrize("case", UNALIGNED_GEMM, ids=lambda c: "L{}m{}n{}k{}".format(*c))
def test_unaligned_rows_gemm(case):
    layout, m, n, k = case
    rng = np.random.default_rng(8400 + m + n + k)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    a = synth.activations(rng, m, k, "bf16")
    c = run_gemm(w, layout, n, k, a, ldc=n + 8 - n % 8)
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c, c_ref, den) <= TOL


@pytest.mark.parametrize("plan", ["main", "tail", "tail2", "tail4", "msplit3"])
@pytest.mark.parametrize("case", [(0, 100, 200, 96), (1, 130, 264, 544), (0, 257, 300, 1376)],
                         ids=lambda c: "L{}m{}n{}k{}".format(*c))
def test_unaligned_rows_gemm_forced_tile_size(case, plan, force):
    """The zero-filled k tail in each tile configuration and in every split part
    (k = 544: 17 blocks, so four splits of the five step pairs)."""
    force(gemm_plan=plan)
    layout, m, n, k = case
    rng = np.random.default_rng(8500 + m + n + k)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    a = synth.activations(rng, m, k, "bf16")
    c = run_gemm(w, layout, n, k, a, ldc=(n + 7) // 8 * 8)
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c, c_ref, den) <= TOL


def test_unaligned_rows_gemm_tail_ignores_values_past_k():
    """A's columns past k are never used: NaN stored in the padding after each row
    (lda > k) does not reach the output of the zero-filled k tail."""
    layout, m, n, k = 0, 65, 96, 160
    lda = k + 8
    rng = np.random.default_rng(8600)
    w = synth.weights(rng, layout, n, k)
    a = synth.activations(rng, m, k, "bf16")
    ad = torch.full((m, lda), float("nan"), dtype=torch.bfloat16, device=DEV)
    ad[:, :k] = a.to(DEV)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    st = R.lib().rfp4_gemm(R._ptr(dev(w)), layout, n, k, R._ptr(ad), m, lda, R._ptr(c), n, R._stream(None))  # noqa
    assert st == R.RFP4_OK
    torch.cuda.synchronize()
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c.to(torch.float64).cpu().numpy(), c_ref, den) <= TOL


@pytest.mark.parametrize("case", [(0, 100, 200, 96), (1, 64, 296, 1056)], ids=lambda c: "L{}m{}n{}k{}".format(*c))
def test_unaligned_rows_gemm_dequant(case):
    layout, m, n, k = case
    rng = np.random.default_rng(8700 + m + n + k)
    w = synth.weights(rng, layout, n, k)
    a = synth.activations(rng, m, k, "bf16")
    wbuf = torch.empty((n, (k + 7) // 8 * 8), dtype=torch.bfloat16, device=DEV)
    c = R.rfp4_gemm_dequant(dev(w), layout, n, k, a.to(DEV).contiguous(), wbuf=wbuf)
    torch.cuda.synchronize()
    c_ref, den = O.gemm(w, layout, n, k, x64(a))
    assert gemm_error(c.to(torch.float64).cpu().numpy(), c_ref, den) <= TOL


# ------------------------------------------------------------------ GEMV on the matrix cores
# Both GEMV kernels are checked at every batch by forcing the path (rfp4_force): "tiles"
# runs the matrix-core kernel (16-row tiles, table decode, k split over the wavefronts of
# a workgroup), "dot" the dot-product kernel. Cases cover ragged row counts, odd block counts
# (single-block units), rows that are not 16-byte multiples, activations staged in LDS and
# read from global memory (long rows, large batches), every wavefront count, and fused
# launches.

MFMA_CASES = [  # layout, n, k, batch, dtype
    (0, 17408, 5120, 1, "f16"), (0, 17408, 5120, 8, "f16"), (1, 5120, 17408, 1, "bf16"),
    (1, 5120, 17408, 8, "bf16"), (0, 6144, 5120, 3, "bf16"), (0, 1024, 5120, 5, "f16"),
    (0, 1, 256, 1, "f16"), (1, 7, 512, 2, "bf16"), (0, 33, 1408, 4, "f16"), (1, 45, 1056, 6, "bf16"),
    (0, 130, 96, 7, "f16"), (1, 17, 32, 8, "bf16"), (0, 300, 4000, 8, "bf16"), (1, 64, 99968, 2, "f16"),
    (0, 999, 2304, 8, "f16"),
    # chunks of 16 units per row: 4 (T % 3 == 1), 7 with a ragged last chunk, 6 with
    # single-block units and a ragged last chunk, 6 exactly at batch 4
    (0, 200, 4096, 4, "f16"), (1, 77, 6912, 5, "bf16"), (0, 50, 2720, 6, "bf16"),
    (1, 5120, 6144, 4, "bf16"),
    # two tiles per workgroup (batch > 4, >= 1024 tiles): n % 32 == 16 leaves the last
    # workgroup's second tile empty; single-block units
    (0, 16400, 512, 6, "f16"), (1, 16400, 1056, 8, "bf16"),
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=lambda c: "L{}n{}k{}b{}{}".format(*c))
def test_gemv_mfma(case, force):
    force(gemv_kernel="tiles")
    layout, n, k, batch, dt = case
    rng = np.random.default_rng(9000 + n + k + batch)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, batch, k, dt)
    check_gemv(w, layout, n, k, x, ldy=n + 3)


@pytest.mark.parametrize("batch", [2, 8])
def test_gemv_dot_product_kernel_large_batch(batch, force):
    force(gemv_kernel="dot")
    w, x, cfg = synth.gemv_inputs("down", batch=batch)
    check_gemv(w, cfg["layout"], cfg["n"], cfg["k"], x)


def test_gemv_mfma_padded_activations(force):
    """ldx > k and ldy > n on the matrix-core path."""
    force(gemv_kernel="tiles")
    layout, n, k, batch = 0, 77, 768, 5
    rng = np.random.default_rng(9100)
    w = synth.weights(rng, layout, n, k)
    x = synth.activations(rng, batch, k, "f16")
    check_gemv(w, layout, n, k, x, ldx=k + 16, ldy=n + 9)


@pytest.mark.parametrize("case", MULTI, ids=lambda c: "L{}p{}k{}b{}{}".format(c[0], len(c[1]), *c[2:]))
def test_gemv_mfma_multi(case, force):
    force(gemv_kernel="tiles")
    layout, ns, k, batch, dt = case
    rng = np.random.default_rng(9200 + sum(ns) + k + batch)
    ws = [synth.weights(rng, layout, n, k, stress_frac=0.01) for n in ns]
    x = synth.activations(rng, batch, k, dt)
    ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, ns, k, x.to(DEV).contiguous())
    torch.cuda.synchronize()
    for w, n, y in zip(ws, ns, ys):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


SPLIT_CASES = [  # layout, n, k, batch, dtype, forced split (reduced to one chunk per part)
    (1, 5120, 17408, 8, "bf16", 2), (1, 5120, 17408, 2, "bf16", 4), (0, 1024, 5120, 3, "f16", 4),
    (0, 33, 1408, 4, "f16", 2), (0, 1, 256, 5, "f16", 4), (1, 45, 1056, 6, "bf16", 4),
    (0, 300, 4000, 8, "bf16", 4), (0, 999, 2304, 7, "f16", 2), (1, 5120, 6144, 4, "bf16", 1),
    (1, 5120, 17408, 8, "bf16", 3), (0, 300, 4000, 6, "f16", 3), (1, 45, 1056, 3, "bf16", 3),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "L{}n{}k{}b{}{}-s{}".format(*c))
def test_gemv_mfma_split(case, force):
    """Each tile's chunks shared by 1 to 4 workgroups whose partial sums meet in the
    stream's workspace; padded output rows stay untouched. Both ways of combining the
    parts (the last part polling for the others, and every part counting itself with the
    last to count adding) match the oracle and each other bitwise."""
    layout, n, k, batch, dt, split = case
    rng = np.random.default_rng(9400 + n + k + batch)
    w = synth.weights(rng, layout, n, k, stress_frac=0.02)
    x = synth.activations(rng, batch, k, dt)
    ys = []
    for combine in (0, 1):
        force(gemv_kernel="tiles", gemv_splits=int(split), gemv_split_combine=combine)
        ys.append(check_gemv(w, layout, n, k, x, ldy=n + 5)[0])
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))


def test_gemv_mfma_split_launch_sequence(force):
    """Launches with different splits and tile counts back to back on one stream, combining
    their parts either way (the arrival counters must be back at zero after each), then
    the first one again."""
    rng = np.random.default_rng(9450)
    shapes = [(0, 700, 2048, 4, 4), (1, 130, 6144, 8, 2), (0, 700, 2048, 4, 3), (0, 64, 5120, 2, 4),
              (0, 700, 2048, 4, 4)]
    data = {}
    for layout, n, k, batch, _ in shapes:
        if (layout, n, k, batch) not in data:
            w = synth.weights(rng, layout, n, k)
            x = synth.activations(rng, batch, k, "f16")
            y_ref, den = O.gemv(w, layout, n, k, x64(x))
            data[(layout, n, k, batch)] = (dev(w), x.to(DEV).contiguous(), y_ref, den)
    ys = []
    for i, (layout, n, k, batch, split) in enumerate(shapes):  # both ways of combining, alternately
        wd, xd, _, _ = data[(layout, n, k, batch)]
        ys.append(R.rfp4_gemv(wd, layout, n, k, xd,
                              force=R.make_force("tiles", gemv_splits=split, gemv_split_combine=i % 2)))
    torch.cuda.synchronize()
    for (layout, n, k, batch, _), y in zip(shapes, ys):
        _, _, y_ref, den = data[(layout, n, k, batch)]
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


def test_gemv_mfma_multi_two_tiles(force):
    """Two matrices fused at batch 7 with enough tiles for two tiles per workgroup: the
    32-row tiles of each part start at the part's first row."""
    force(gemv_kernel="tiles")
    layout, ns, k, batch = 0, [9000, 8008], 256, 7
    rng = np.random.default_rng(9470)
    ws = [synth.weights(rng, layout, n, k, stress_frac=0.01) for n in ns]
    x = synth.activations(rng, batch, k, "f16")
    ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, ns, k, x.to(DEV).contiguous())
    torch.cuda.synchronize()
    for w, n, y in zip(ws, ns, ys):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


def test_gemv_mfma_multi_split(force):
    force(gemv_kernel="tiles", gemv_splits=4)
    layout, ns, k, batch = 1, [300, 45, 1000, 7], 6144, 5
    rng = np.random.default_rng(9460)
    ws = [synth.weights(rng, layout, n, k, stress_frac=0.01) for n in ns]
    x = synth.activations(rng, batch, k, "bf16")
    ys = R.rfp4_gemv_multi([dev(w) for w in ws], layout, ns, k, x.to(DEV).contiguous())
    torch.cuda.synchronize()
    for w, n, y in zip(ws, ns, ys):
        y_ref, den = O.gemv(w, layout, n, k, x64(x))
        assert O.normalized_error(y.cpu().numpy(), y_ref, den) <= TOL


def test_gemv_mfma_zero_scales_give_zero(force):
    force(gemv_kernel="tiles")
    layout, n, k, batch = 0, 40, 512, 4
    w = synth.weights(np.random.default_rng(9300), layout, n, k).reshape(n, k // 32, 18)
    w[:, :, 16:] = 0
    x = synth.activations(np.random.default_rng(9301), batch, k, "bf16")
    y = run_gemv(w.reshape(n, -1), layout, n, k, x)
    assert np.all(y == 0.0)


# ------------------------------------------------------------------ graph capture

def test_graph_replay_matches_eager(force):
    """Every entry point captured into one HIP graph (batch-1 and batch-4 GEMV, a
    batch-4 GEMV on long rows whose tiles split, fused two-matrix GEMVs at batch 1 and
    4, a GEMM with split k, dequant, encoder)
    and replayed three times, with eager work between the replays, gives exactly the
    eager results. Everything runs on the capture stream first so that the workspaces
    exist before the capture, as the header asks."""
    force(gemm_plan="tail2")
    rng = np.random.default_rng(9500)
    layout, n, k = 0, 1040, 2048
    wd = dev(synth.weights(rng, layout, n, k))
    x1 = synth.activations(rng, 1, k, "f16").to(DEV).contiguous()
    x4 = synth.activations(rng, 4, k, "bf16").to(DEV).contiguous()
    a = synth.activations(rng, 200, k, "bf16").to(DEV).contiguous()
    src = synth.real_weights(rng, 96, k, "bf16").to(DEV).contiguous()

    ws_layout, ws_n, ws_k = 1, 520, 12288  # long rows: the batch-4 GEMV splits its tiles
    wsd = dev(synth.weights(rng, ws_layout, ws_n, ws_k))
    xs4 = synth.activations(rng, 4, ws_k, "bf16").to(DEV).contiguous()
    mn = [300, 170]  # fused parts sharing the activations
    wms = [dev(synth.weights(rng, layout, m, k)) for m in mn]
    outs = {"ys": torch.empty((4, ws_n), dtype=torch.float32, device=DEV),
            "m1a": torch.empty((1, mn[0]), dtype=torch.float32, device=DEV),
            "m1b": torch.empty((1, mn[1]), dtype=torch.float32, device=DEV),
            "m4a": torch.empty((4, mn[0]), dtype=torch.float32, device=DEV),
            "m4b": torch.empty((4, mn[1]), dtype=torch.float32, device=DEV),
            "y1": torch.empty((1, n), dtype=torch.float32, device=DEV),
            "y4": torch.empty((4, n), dtype=torch.float32, device=DEV),
            "c": torch.empty((200, n), dtype=torch.bfloat16, device=DEV),
            "d": torch.empty((n, k), dtype=torch.float32, device=DEV),
            "q": torch.empty((96, R.rfp4_row_bytes(layout, k)), dtype=torch.uint8, device=DEV)}

    def run():
        R.rfp4_gemv(wsd, ws_layout, ws_n, ws_k, xs4, y=outs["ys"])
        R.rfp4_gemv(wd, layout, n, k, x1, y=outs["y1"])
        R.rfp4_gemv(wd, layout, n, k, x4, y=outs["y4"])
        R.rfp4_gemv_multi(wms, layout, mn, k, x1, [outs["m1a"], outs["m1b"]])
        R.rfp4_gemv_multi(wms, layout, mn, k, x4, [outs["m4a"], outs["m4b"]])
        R.rfp4_gemm(wd, layout, n, k, a, c=outs["c"])
        R.rfp4_dequant(wd, layout, n, k, out=outs["d"])
        R.rfp4_quantize(src, layout, out=outs["q"])

    run()
    torch.cuda.synchronize()
    eager = {key: v.clone() for key, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capture stream (its GEMM workspace)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    for rep in range(3):
        for v in outs.values():
            v.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, v in outs.items():
            assert torch.equal(v, eager[key]), (key, rep)


def test_gemv_split_two_streams(force):
    """Split-tile GEMVs interleaved on two streams: each stream has its own workspace
    (partial sums and arrival counters), so concurrent launches do not mix."""
    force(gemv_kernel="tiles", gemv_splits=2)
    rng = np.random.default_rng(9600)
    layout, n, k = 1, 640, 12288
    ws = [synth.weights(rng, layout, n, k) for _ in range(2)]
    xs = [synth.activations(rng, 4, k, "bf16") for _ in range(2)]
    wds = [dev(w) for w in ws]
    xds = [x.to(DEV).contiguous() for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ys = [[torch.empty((4, n), dtype=torch.float32, device=DEV) for _ in range(6)] for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(6):
        for s in range(2):
            with torch.cuda.stream(streams[s]):
                R.rfp4_gemv(wds[s], layout, n, k, xds[s], y=ys[s][rep])
    torch.cuda.synchronize()
    for s in range(2):
        y_ref, den = O.gemv(ws[s], layout, n, k, x64(xs[s]))
        for rep in range(6):
            assert O.normalized_error(ys[s][rep].cpu().numpy(), y_ref, den) <= TOL
            assert torch.equal(ys[s][rep], ys[s][0])


@pytest.mark.parametrize("mode,batch", [("dot", 1), ("tall", 1), ("tiles", 4), ("tiles", 8)])
def test_gemv_vocab_rows_sampled(mode, batch, force):
    """A vocabulary-sized matrix (152064 x 5120 dual, 438 MB packed: the decode LM head)
    on each kernel (batch 1: the dot-product kernel, the default for one matrix, and the
    tall matrix-core kernel; batches 4 and 8 on the matrix-core tiles), checked on a
    seeded sample of rows that includes the first and the last."""
    force(gemv_kernel=mode)
    layout, n, k = 0, 152064, 5120
    rng = np.random.default_rng(9700 + batch)
    w = synth.weights(rng, layout, n, k)
    x = synth.activations(rng, batch, k, "f16")
    y = R.rfp4_gemv(dev(w), layout, n, k, x.to(DEV).contiguous()).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.choice(n, 96, replace=False)]))
    y_ref, den = O.gemv_rows(w, layout, n, k, x64(x), rows)
    assert O.normalized_error(y[:, rows], y_ref, den) <= TOL


def test_workspace_growth_keeps_captured_graphs_valid():
    """A graph captured with a split GEMM and a split-tile GEMV, then eager calls on the
    same stream with larger shapes (the GEMM's partial sums outgrow the stream's
    workspace, so the library moves to a larger buffer and keeps the old one), then
    replays with more eager work between them: every replay gives the eager results of
    the captured shapes bit for bit, and the larger calls stay correct."""
    rng = np.random.default_rng(9800)
    fg = R.make_force(gemm_plan="tail2")
    fv = R.make_force("tiles", gemv_splits=2)
    layout, n, k = 0, 1040, 2048
    wd = dev(synth.weights(rng, layout, n, k))
    a = synth.activations(rng, 200, k, "bf16").to(DEV).contiguous()
    vl, vn, vk = 1, 520, 12288
    wv = dev(synth.weights(rng, vl, vn, vk))
    xv = synth.activations(rng, 4, vk, "bf16").to(DEV).contiguous()
    big_w = synth.weights(rng, layout, 4096, k)
    big_a = synth.activations(rng, 1024, k, "bf16")
    big_wd, big_ad = dev(big_w), big_a.to(DEV).contiguous()
    big_vw = synth.weights(rng, vl, 1000, vk)
    big_vx = synth.activations(rng, 8, vk, "bf16")
    big_vwd, big_vxd = dev(big_vw), big_vx.to(DEV).contiguous()
    c = torch.empty((200, n), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((4, vn), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        R.rfp4_gemm(wd, layout, n, k, a, c, force=fg)  # creates the stream's workspaces
        R.rfp4_gemv(wv, vl, vn, vk, xv, y, force=fv)
        s.synchronize()
        eager_c, eager_y = c.clone(), y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            R.rfp4_gemm(wd, layout, n, k, a, c, force=fg)
            R.rfp4_gemv(wv, vl, vn, vk, xv, y, force=fv)
        big_c = R.rfp4_gemm(big_wd, layout, 4096, k, big_ad, force=fg)  # outgrows the workspace
        big_y = R.rfp4_gemv(big_vwd, vl, 1000, vk, big_vxd, force=fv)
        s.synchronize()
        for rep in range(3):
            c.zero_()
            y.zero_()
            g.replay()
            R.rfp4_gemm(big_wd, layout, 4096, k, big_ad, big_c, force=fg)
            s.synchronize()
            assert torch.equal(c, eager_c), rep
            assert torch.equal(y, eager_y), rep
    c_ref, den = O.gemm(big_w, layout, 4096, k, x64(big_a))
    assert gemm_error(big_c.to(torch.float64).cpu().numpy(), c_ref, den) <= TOL
    y_ref, vden = O.gemv(big_vw, vl, 1000, vk, x64(big_vx))
    assert O.normalized_error(big_y.cpu().numpy(), y_ref, vden) <= TOL


CAPTURE_FIRST_SCRIPT = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import gemm_rfp4_block_amd as R, synth
import oracle.rfp4_oracle as O
dev = torch.device("cuda:0")
rng = np.random.default_rng(9800)
layout, n, k = 1, 520, 12288  # 33 tiles, 12 chunks per row: two parts from batch 3
w = synth.weights(rng, layout, n, k)
wd = torch.from_numpy(w).to(dev)
x3 = synth.activations(rng, 3, k, "bf16").to(dev).contiguous()
x8 = synth.activations(rng, 8, k, "bf16").to(dev).contiguous()
side = torch.cuda.Stream()
side.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(side):
    R.rfp4_gemv(wd, layout, n, k, x3)  # the stream's workspace, and the batch-3 tile kernel only
torch.cuda.current_stream().wait_stream(side)
torch.cuda.synchronize()
y8 = torch.empty((8, n), dtype=torch.float32, device=dev)
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=side):
    R.rfp4_gemv(wd, layout, n, k, x8, y=y8)  # first launch of the batch-8 kernel: under capture
outs = []
for _ in range(3):
    y8.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    outs.append(y8.clone())
eager = R.rfp4_gemv(wd, layout, n, k, x8)
torch.cuda.synchronize()
y_ref, den = O.gemv(w, layout, n, k, x8.cpu().double().numpy())
for o in outs:
    assert torch.equal(o, outs[0])
    assert O.normalized_error(o.cpu().numpy(), y_ref, den) <= 2e-3
assert torch.equal(outs[0], eager), "replay differs from the eager call"
print("capture-first ok")
"""


def test_first_split_launch_of_a_kernel_under_graph_capture():
    """In a fresh process, the first launch of a split tile kernel at batch 8 (its
    occupancy, which the split count depends on, not yet known) happens inside a graph
    capture on a stream whose split workspace a batch-3 launch has already allocated: the
    capture succeeds, and every replay gives the eager result bitwise and matches the
    oracle."""
    import subprocess
    import sys

    from tests.conftest import ROOT
    r = subprocess.run([sys.executable, "-c", CAPTURE_FIRST_SCRIPT, ROOT], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "capture-first ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
