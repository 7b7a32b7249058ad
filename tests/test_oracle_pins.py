"""Pins of the CPU oracle to facts outside itself (CPU only).

Each ``check_*`` function raises AssertionError when the oracle disagrees with:
the block sizes and codebook printed on "Feasibility Report: Porting ROCmFP4 to
Atlas" (subsections "Block Layout", "Codebook10 Value Table"); the textbook E4M3
encoding and torch's float8_e4m3fn; exact rational arithmetic on tiny matrices;
special cases that reduce to integer matrix products; and exact invariants. The
mutation test at the end plants plausible mistakes in the oracle and checks that
each one trips at least one pin.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.rfp4_oracle as O
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


FACTS = _load("format_facts.json")
E4M3 = _load("e4m3_textbook.json")
WITNESS = _load("witness_blocks.json")
PRINTED_CB = FACTS["codebook10"]["values"]
LAYOUTS = {"dual": O.DUAL, "fast": O.FAST}


# ---------------------------------------------------------------- helpers (test-owned)

def torch_e4m3_magnitude(u7: int) -> Fraction:
    """E4M3 magnitude of a 7-bit field through torch's float8_e4m3fn (library routine)."""
    v = torch.tensor([u7], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
    return Fraction(v)


def pack_blocks(idx: np.ndarray, sbytes: np.ndarray, layout: int) -> np.ndarray:
    """Test-owned packer: idx (n, nb, 32) ints 0..15, sbytes (n, nb, ns) -> bytes (n, row)."""
    n, nb, _ = idx.shape
    qs = (idx[:, :, :16] | (idx[:, :, 16:] << 4)).astype(np.uint8)
    blocks = np.concatenate([qs, sbytes.astype(np.uint8)], axis=2)
    return blocks.reshape(n, -1)


def exact_weights(idx, sbytes, layout):
    """Exact rational weight of every element from the printed codebook and torch's E4M3."""
    n, nb, _ = idx.shape
    out = [[None] * (nb * 32) for _ in range(n)]
    for r in range(n):
        for j in range(nb):
            for t in range(32):
                if layout == O.DUAL:
                    b = int(sbytes[r, j, 0 if t < 16 else 1])
                else:
                    b = int(sbytes[r, j, 0])
                s = torch_e4m3_magnitude(b & 0x7F) / 2
                out[r][32 * j + t] = Fraction(PRINTED_CB[int(idx[r, j, t])]) * s
    return out


def random_case(rng, layout, n, k, exp_lo=0, exp_hi=15):
    nb = k // 32
    ns = 2 if layout == O.DUAL else 1
    idx = rng.integers(0, 16, size=(n, nb, 32))
    ex = rng.integers(exp_lo, exp_hi + 1, size=(n, nb, ns))
    mu = rng.integers(0, 8, size=(n, nb, ns))
    sb = (ex << 3) | mu
    sb = np.where((sb & 0x7F) == 0x7F, 0x7E, sb)  # finite bytes only
    sb = sb | (rng.integers(0, 2, size=sb.shape) << 7)  # bit 7 ignored by reading R-SIGN
    return idx, sb


def fp16_vector(rng, rows, k):
    return rng.standard_normal((rows, k)).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------- checks

def check_block_layout():
    bl = FACTS["block_layout"]
    for name, lay in LAYOUTS.items():
        assert O.block_bytes(lay) == bl[name]["block_bytes"]
        assert O.block_bytes(lay) == bl[name]["qs_bytes"] + bl[name]["scale_bytes"]
        assert O.bits_per_weight(lay) == bl[name]["bits_per_weight"]
        assert O.row_bytes(lay, 512) == 16 * bl[name]["block_bytes"]


def check_codebook():
    assert list(O.CODEBOOK10) == PRINTED_CB
    cb = np.array(PRINTED_CB)
    assert np.all(cb[8:] == -cb[:8])  # index bit 3 is the sign
    e2m1 = FACTS["e2m1"]
    assert list(cb[:7]) == [2 * v for v in e2m1["grid"][:7]]
    assert 2 * e2m1["grid"][7] == e2m1["retuned_largest_from"]
    assert cb[7] == e2m1["retuned_largest_to"]


def check_e4m3():
    vals = O.e4m3_value(np.arange(128))
    for p in E4M3["points"]:
        assert vals[p["byte"]] == p["value"], p
    for b in range(256):
        t = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
        if b in E4M3["nan_bytes"]:
            assert np.isnan(t)
            assert O.e4m3_value(b & 0x7F) == 480.0  # reading R-NAN
            continue
        assert abs(t) == O.e4m3_value(b & 0x7F), b


def check_scale():
    s = O.scale_value(np.arange(256))
    assert s[0x40] == 1.0
    assert np.array_equal(s[:128], s[128:])  # reading R-SIGN
    assert np.array_equal(s[:128], O.e4m3_value(np.arange(128)) / 2)  # reading R-HALF
    for b in range(8, 120):  # exponent fields 1..14
        assert s[b + 8] == 2 * s[b], b
    assert s[0x7F] == 240.0


def check_witness():
    qs = np.frombuffer(bytes.fromhex(WITNESS["qs_hex"]), dtype=np.uint8)
    for blk in WITNESS["blocks"]:
        lay = LAYOUTS[blk["layout"]]
        w = np.concatenate([qs, np.array(blk["scales"], dtype=np.uint8)]).reshape(1, -1)
        got = O.dequantize_f32(w, lay, 1, 32)[0]
        exp = np.array(blk["expected"], dtype=np.float32)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), blk["note"]


def check_fraction_dequant_and_gemv(seed=1):
    rng = np.random.default_rng(seed)
    for lay in (O.DUAL, O.FAST):
        for (n, k, batch) in ((3, 64, 1), (4, 96, 3), (2, 32, 2)):
            idx, sb = random_case(rng, lay, n, k)
            w = pack_blocks(idx, sb, lay)
            ex_w = exact_weights(idx, sb, lay)
            got_w = O.dequantize(w, lay, n, k)
            for r in range(n):
                for c in range(k):
                    assert Fraction(got_w[r, c]) == ex_w[r][c], (lay, r, c)
            x = fp16_vector(rng, batch, k)
            y, den = O.gemv(w, lay, n, k, x)
            assert y.shape == (batch, n)
            for b in range(batch):
                for r in range(n):
                    ex = sum(ex_w[r][c] * Fraction(x[b, c]) for c in range(k))
                    ab = sum(abs(ex_w[r][c] * Fraction(x[b, c])) for c in range(k))
                    assert abs(Fraction(y[b, r]) - ex) <= Fraction(k, 2 ** 52) * ab, (lay, b, r)
                    assert Fraction(den[b, r]) == ab or abs(Fraction(den[b, r]) - ab) <= Fraction(k, 2 ** 52) * ab


def check_fraction_gemm(seed=2):
    rng = np.random.default_rng(seed)
    for lay in (O.DUAL, O.FAST):
        n, k, m = 3, 64, 4
        idx, sb = random_case(rng, lay, n, k)
        w = pack_blocks(idx, sb, lay)
        ex_w = exact_weights(idx, sb, lay)
        a = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16).double().numpy()
        c, den = O.gemm(w, lay, n, k, a)
        assert c.shape == (m, n)
        for i in range(m):
            for r in range(n):
                ex = sum(Fraction(a[i, q]) * ex_w[r][q] for q in range(k))
                ab = sum(abs(Fraction(a[i, q]) * ex_w[r][q]) for q in range(k))
                assert abs(Fraction(c[i, r]) - ex) <= Fraction(k, 2 ** 52) * ab


def check_special_cases(seed=3):
    rng = np.random.default_rng(seed)
    n, k = 5, 128
    for lay in (O.DUAL, O.FAST):
        ns = 2 if lay == O.DUAL else 1
        idx = rng.integers(0, 16, size=(n, k // 32, 32))
        sb = np.full((n, k // 32, ns), 0x40)  # every scale decodes to 1
        w = pack_blocks(idx, sb, lay)
        intmat = np.array(PRINTED_CB)[idx].reshape(n, k)
        x = fp16_vector(rng, 2, k)
        y, _ = O.gemv(w, lay, n, k, x)
        assert np.array_equal(y, x @ intmat.T.astype(np.float64))
        for j in (0, 17, 31, 32, 100):  # one-hot x picks a column
            e = np.zeros((1, k))
            e[0, j] = 1.0
            y1, _ = O.gemv(w, lay, n, k, e)
            assert np.array_equal(y1[0], intmat[:, j].astype(np.float64))
        ones = pack_blocks(np.ones_like(idx), sb, lay)  # all codes +1
        y2, _ = O.gemv(ones, lay, n, k, x)
        assert np.allclose(y2, np.repeat(x.sum(axis=1, keepdims=True), n, axis=1), rtol=0, atol=1e-12)


def check_invariants(seed=4):
    rng = np.random.default_rng(seed)
    n, k = 6, 256
    for lay in (O.DUAL, O.FAST):
        bb = O.block_bytes(lay)
        idx, sb = random_case(rng, lay, n, k, exp_lo=1, exp_hi=13)
        w = pack_blocks(idx, sb, lay)
        x = fp16_vector(rng, 2, k)
        y, _ = O.gemv(w, lay, n, k, x)
        blocks = w.reshape(n, k // 32, bb).copy()
        flip = blocks.copy()
        flip[:, :, :16] ^= 0x88  # toggle the sign bit of every index
        yf, _ = O.gemv(flip.reshape(n, -1), lay, n, k, x)
        assert np.array_equal(yf, -y)
        step = blocks.copy()
        step[:, :, 16:] += 8  # exponent field + 1
        ys, _ = O.gemv(step.reshape(n, -1), lay, n, k, x)
        assert np.array_equal(ys, 2 * y)
    # dual with equal half scales == fast with that scale
    idx, sb = random_case(rng, O.FAST, n, k)
    wf = pack_blocks(idx, sb, O.FAST)
    wd = pack_blocks(idx, np.concatenate([sb, sb], axis=2), O.DUAL)
    a = O.dequantize_f32(wf, O.FAST, n, k)
    b = O.dequantize_f32(wd, O.DUAL, n, k)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def check_gemm_orientation(seed=5):
    """C = A W^T: row m of C is the GEMV of row m of A."""
    rng = np.random.default_rng(seed)
    n, k, m = 7, 64, 3
    idx, sb = random_case(rng, O.DUAL, n, k)
    w = pack_blocks(idx, sb, O.DUAL)
    a = fp16_vector(rng, m, k)
    c, _ = O.gemm(w, O.DUAL, n, k, a)
    y, _ = O.gemv(w, O.DUAL, n, k, a)
    assert c.shape == (m, n) and np.array_equal(c, y)


def unpack_blocks(w: np.ndarray, layout: int, n: int, k: int):
    """Test-owned unpacker (inverse of pack_blocks): (idx (n, nb, 32), sbytes (n, nb, ns))."""
    nb = k // 32
    bb = 18 if layout == O.DUAL else 17
    blk = np.asarray(w, dtype=np.uint8).reshape(n, nb, bb).astype(np.int64)
    idx = np.concatenate([blk[:, :, :16] & 15, blk[:, :, :16] >> 4], axis=2)
    return idx, blk[:, :, 16:]


def check_quantize_roundtrip(seed=6):
    """Encoding the exact values of blocks whose every scale group holds a +-10 code (and no
    index 8, the second zero) gives back the same bytes: the encoder inverts the
    printed codebook, torch's E4M3 and the nibble convention."""
    rng = np.random.default_rng(seed)
    for layout in (O.DUAL, O.FAST):
        n, k = 5, 256
        nb, g = k // 32, (16 if layout == O.DUAL else 32)
        ns = 32 // g
        idx = rng.choice([i for i in range(16) if i != 8], size=(n, nb, 32))
        for r in range(n):
            for j in range(nb):
                for h in range(ns):
                    idx[r, j, h * g + rng.integers(0, g)] = rng.choice([7, 15])
        sb = rng.integers(1, 127, size=(n, nb, ns))
        w = pack_blocks(idx, sb, layout)
        vals = np.array([[float(v) for v in row] for row in exact_weights(idx, sb, layout)])
        assert np.array_equal(O.quantize(vals, layout), w)


def check_quantize_nearest_minimal(seed=7):
    """Brute force on random values, exact ties and extremes: each group's scale is the
    smallest finite one that reaches its largest magnitude with code 10, and each weight's
    code is the codebook entry nearest to it (ties to the smaller magnitude, zero as
    index 0). Exact rational arithmetic throughout."""
    rng = np.random.default_rng(seed)
    for layout in (O.DUAL, O.FAST):
        n, k = 4, 128
        v = rng.standard_normal((n, k)) * np.exp2(rng.integers(-12, 12, size=(n, 1)))
        v[0, :32] = 0.0
        v[0, 5] = -0.0
        v[1, :32] = np.float32(1e6) * np.sign(rng.standard_normal(32))
        s3 = 0.5 * float(torch_e4m3_magnitude(0x3B))  # a normal scale
        ties = np.array([0.5, 1.5, 2.5, 3.5, 5.0, 7.0, 9.0, 10.0, -0.5, -9.0, 4.0, -6.0, 1.0, 2.0, 3.0, 8.0])
        v[2, :32] = np.concatenate([ties, -ties]) * s3
        v[3, :32] = 1e-30 * np.arange(32)
        q = O.quantize(v, layout)
        idx, sb = unpack_blocks(q, layout, n, k)
        g = 16 if layout == O.DUAL else 32
        half = [Fraction(0)] + [torch_e4m3_magnitude(u) / 2 for u in range(1, 127)]
        for r in range(n):
            for j in range(k // 32):
                for h in range(32 // g):
                    b = int(sb[r, j, h])
                    assert b <= 126
                    grp = [Fraction(float(x)) for x in v[r, 32 * j + h * g: 32 * j + (h + 1) * g]]
                    amax = max(abs(x) for x in grp)
                    if amax <= 10 * half[126]:
                        assert 10 * half[b] >= amax and (b == 0 or 10 * half[b - 1] < amax)
                    else:
                        assert b == 126
                    S = half[b]
                    for t, x in enumerate(grp):
                        i = int(idx[r, j, h * g + t])
                        best = min(range(16), key=lambda c: (abs(x - PRINTED_CB[c] * S), abs(PRINTED_CB[c]), c))
                        assert abs(x - PRINTED_CB[i] * S) == abs(x - PRINTED_CB[best] * S)
                        assert abs(PRINTED_CB[i]) == abs(PRINTED_CB[best])
                        if PRINTED_CB[i] == 0:
                            assert i == 0
                        else:
                            assert (i >= 8) == (x < 0)


ALL_CHECKS = [check_block_layout, check_codebook, check_e4m3, check_scale, check_witness,
              check_fraction_dequant_and_gemv, check_fraction_gemm, check_special_cases,
              check_invariants, check_gemm_orientation, check_quantize_roundtrip,
              check_quantize_nearest_minimal]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


# ---------------------------------------------------------------- validation, misc

def test_validate_rejects_nonfinite_scales():
    rng = np.random.default_rng(7)
    for lay in (O.DUAL, O.FAST):
        n, k = 4, 256
        ns = 2 if lay == O.DUAL else 1
        bb = O.block_bytes(lay)
        idx, sb = random_case(rng, lay, n, k)
        w = pack_blocks(idx, sb, lay)
        w[:, :16] = 0x7F  # index bytes never matter
        assert O.validate(w, lay, n, k) == (True, -1)
        bad = w.reshape(n, k // 32, bb).copy()
        bad[1, 3, 16 + ns - 1] = 0xFF
        bad[2, 0, 16] = 0x7F
        assert O.validate(bad.reshape(n, -1), lay, n, k) == (False, 1 * (k // 32) + 3)
        ok = w.reshape(n, k // 32, bb).copy()
        ok[0, 0, 16] = 0xFE  # largest finite with bit 7 set
        assert O.validate(ok.reshape(n, -1), lay, n, k) == (True, -1)


def test_normalized_error_semantics():
    assert O.normalized_error([1.0, 0.0], [1.0, 0.0], [2.0, 0.0]) == 0.0
    assert O.normalized_error([1.5], [1.0], [2.0]) == 0.25
    assert O.normalized_error([1e-30], [0.0], [0.0]) == float("inf")


def test_rows_helpers_match_full():
    rng = np.random.default_rng(8)
    n, k = 9, 128
    idx, sb = random_case(rng, O.DUAL, n, k)
    w = pack_blocks(idx, sb, O.DUAL)
    x = fp16_vector(rng, 2, k)
    y, den = O.gemv(w, O.DUAL, n, k, x)
    rows = np.array([0, 4, 8])
    yr, dr = O.gemv_rows(w, O.DUAL, n, k, x, rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(dr, den[:, rows])
    c, _ = O.gemm(w, O.DUAL, n, k, x)
    cr, _ = O.gemm_rows(w, O.DUAL, n, k, x, rows)
    assert np.array_equal(cr, c[:, rows])


# ---------------------------------------------------------------- planted mistakes

def _mut_sequential_nibbles(qs):
    lo = qs & 0x0F
    hi = qs >> 4
    return np.stack([lo, hi], axis=-1).reshape(*qs.shape[:-1], 32).astype(np.int64)


def _mut_swapped_planes(qs):
    return np.concatenate([qs >> 4, qs & 0x0F], axis=-1).astype(np.int64)


def _mut_no_half(b):
    return O.e4m3_value(np.asarray(b, dtype=np.int64) & 0x7F)


def _mut_sign_kept(b):
    b = np.asarray(b, dtype=np.int64)
    return 0.5 * O.e4m3_value(b & 0x7F) * np.where(b & 0x80, -1.0, 1.0)


def _mut_subnormal_as_normal(u):
    u = np.asarray(u, dtype=np.int64)
    return np.ldexp(1.0 + (u & 7) / 8.0, ((u >> 3) - 7).astype(np.int64))


def _mut_bias8(u):
    u = np.asarray(u, dtype=np.int64)
    e, m = u >> 3, u & 7
    return np.where(e == 0, m * 2.0 ** -10, np.ldexp(1.0 + m / 8.0, (e - 8).astype(np.int64)))


def _mut_dual_one_scale(e, layout):
    s = O.scale_value(e)
    return np.repeat(s[..., :1], 32, axis=-1)


def _mut_dual_halves_swapped(e, layout):
    s = O.scale_value(e)
    if layout == O.DUAL:
        s = s[..., ::-1]
        return np.repeat(s, 16, axis=-1)
    return np.repeat(s, 32, axis=-1)


def _mut_gemv_abs_missing(w, layout, n, k, x):
    wd = O.dequantize(w, layout, n, k)
    x = np.asarray(x, dtype=np.float64).reshape(-1, k)
    return x @ np.abs(wd).T, np.abs(x) @ np.abs(wd).T


def _mut_gemv_reversed_k(w, layout, n, k, x):
    wd = O.dequantize(w, layout, n, k)
    x = np.asarray(x, dtype=np.float64).reshape(-1, k)
    return x[:, ::-1] @ wd.T, np.abs(x) @ np.abs(wd).T


def _mut_gemm_dropped_block(w, layout, n, k, a):
    wd = O.dequantize(w, layout, n, k).copy()
    wd[:, -32:] = 0.0
    a = np.asarray(a, dtype=np.float64)
    return a @ wd.T, np.abs(a) @ np.abs(wd).T


def _mut_quant_ties_up(v, layout):
    """Ties go to the larger magnitude."""
    eps = 1e-12
    return _orig_quantize(np.asarray(v, dtype=np.float64) * (1 + eps), layout)


def _mut_quant_scale_one_up(v, layout):
    q = _orig_quantize(v, layout).copy()
    n, k = np.asarray(v).shape
    bb = 18 if layout == O.DUAL else 17
    blk = q.reshape(n, k // 32, bb)
    blk[:, :, 16:] = np.minimum(blk[:, :, 16:] + 1, 126)
    return q


def _mut_quant_planes_swapped(v, layout):
    q = _orig_quantize(v, layout).copy()
    n, k = np.asarray(v).shape
    bb = 18 if layout == O.DUAL else 17
    blk = q.reshape(n, k // 32, bb)
    blk[:, :, :16] = (blk[:, :, :16] >> 4) | ((blk[:, :, :16] & 15) << 4)
    return q


_orig_quantize = O.quantize

MUTATIONS = {
    "quant_midpoint_5_to_5.5": ("MIDPOINTS", (0.5, 1.5, 2.5, 3.5, 5.5, 7.0, 9.0)),
    "quant_allows_nonfinite_byte": ("MAX_FINITE_SCALE_BYTE", 127),
    "quant_ties_to_larger": ("quantize", _mut_quant_ties_up),
    "quant_scale_one_step_up": ("quantize", _mut_quant_scale_one_up),
    "quant_nibble_planes_swapped": ("quantize", _mut_quant_planes_swapped),
    "sequential_nibbles": ("nibble_indices", _mut_sequential_nibbles),
    "swapped_nibble_planes": ("nibble_indices", _mut_swapped_planes),
    "codebook_12": ("CODEBOOK10", np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12])),
    "codebook_sign_swapped": ("CODEBOOK10", -O.CODEBOOK10),
    "codebook_e2m1": ("CODEBOOK10", np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 0, -0.5, -1, -1.5, -2, -3, -4, -6])),
    "scale_not_halved": ("scale_value", _mut_no_half),
    "scale_bit7_as_sign": ("scale_value", _mut_sign_kept),
    "subnormal_as_normal": ("e4m3_value", _mut_subnormal_as_normal),
    "exponent_bias_8": ("e4m3_value", _mut_bias8),
    "dual_uses_first_scale": ("per_weight_scale", _mut_dual_one_scale),
    "dual_halves_swapped": ("per_weight_scale", _mut_dual_halves_swapped),
    "gemv_sign_dropped": ("gemv", _mut_gemv_abs_missing),
    "gemv_index_reversed": ("gemv", _mut_gemv_reversed_k),
    "gemm_last_block_dropped": ("gemm", _mut_gemm_dropped_block),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, repl = MUTATIONS[name]
    monkeypatch.setattr(O, attr, repl)
    caught = []
    for check in ALL_CHECKS:
        try:
            check()
        except AssertionError:
            caught.append(check.__name__)
        except Exception:  # a crash (shape error etc.) also counts as detection
            caught.append(check.__name__ + "!")
    assert caught, f"mutation {name} slipped past every pin"
