"""ROCmFP4 CPU oracle: plain, slow, fp64 NumPy.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or load this
module: only the test suite (tests/), ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code, table or helper with the HIP library
under ``gemm_rfp4_block_amd/``; the only code both sides use is the seeded input
generator package ``synth/``, which holds none of the method's arithmetic.

What it computes comes from one web page, "Feasibility Report: Porting ROCmFP4 to
Atlas", section "What is ROCmFP4?", subsections:

* "Block Layout" -- a block holds 32 weights: 16 bytes ``qs`` of packed 4-bit
  indices followed by two scale bytes (dual-scale, 18 B, 4.50 bits/weight; one
  scale per 16-weight half) or one scale byte (fast single-scale, 17 B, 4.25
  bits/weight).
* "Codebook10 Value Table" -- the 16 signed integers an index selects; the high bit
  of the index is the sign, and the largest magnitude is 10 rather than the 12 that a
  doubled E2M1 grid would give.
* "Scale Format" -- the scale bytes are finite unsigned E4M3, decoded to half-scale
  fp32 values straight from the exponent and mantissa bits; non-finite bytes are
  rejected once, by row validation, so the decoder never sees them.

The page does not fix: the order of the 32 nibbles inside ``qs``, the exact
meaning of "half-scale", the treatment of an E4M3 exponent field of zero, of bit 7 of
a scale byte, of the two bytes whose low seven bits are all ones, the sign of a
zero weight, the order of blocks in a matrix, nor the output precision. The readings
taken here (each also listed with its reason in the design notes):

  R-NIB   index t (t < 16) is the low nibble of qs[t]; index t + 16 is its high
          nibble, so each 16-weight half is one nibble plane.   [parity unpinned]
  R-HALF  decoded scale S(b) = E4M3(b & 0x7F) / 2.                [parity unpinned]
  R-SUB   exponent field 0 is the textbook E4M3 subnormal, mantissa * 2**-9.
  R-SIGN  bit 7 of a scale byte is ignored by the decoder ("unsigned").
  R-NAN   0x7F / 0xFF are rejected by ``validate``; if decoded anyway they follow
          the bit formula (E4M3 = 480, S = 240), never NaN.
  R-ZERO  a weight is the IEEE product codebook[idx] * S, so a negative code times a
          zero scale is -0.0.
  R-ROW   a matrix of N rows x K columns is N rows of K/32 consecutive blocks; block j
          of a row covers columns 32j .. 32j+31; rows are packed back to back.
  R-OUT   GEMV output fp32, GEMM output bf16 (rounded to nearest even); both
          accumulate in fp32 on the device. The oracle computes the exact result in fp64.
  R-QUANT the encoder (``quantize``): smallest finite half-scale reaching the group's
          largest magnitude with code 10, then the nearest codebook entry, ties to the
          smaller magnitude. The page gives no encoder; pinned by the decode round trip
          and by brute-force nearest-entry and minimal-scale checks. [parity unpinned]

Pins (tests under tests/ marked "not gpu"): the printed block sizes and bits per
weight, the printed codebook, E4M3 on all 256 bytes against the textbook closed form
and against torch's float8_e4m3fn, exact rational brute force on tiny matrices, the
special cases that reduce to an integer matrix product, and exact invariants (sign
flip, exponent step, dual == fast when both halves share a scale). The three readings
marked "parity unpinned" cannot be checked against the page: R-NIB and R-HALF are
pinned only to their own stated convention through witness blocks, R-QUANT to its
stated rule by exact brute force.
"""

from __future__ import annotations

import numpy as np

DUAL = 0  # Q4_0_ROCMFP4: qs[16] + e[2]   ("Block Layout")
FAST = 1  # Q4_0_ROCMFP4_FAST: qs[16] + e ("Block Layout")

WEIGHTS_PER_BLOCK = 32
QS_BYTES = 16

# "Codebook10 Value Table": index 0..7 are the non-negative values, 8..15 their
# negatives (index bit 3 is the sign; index 8 is a second zero).
CODEBOOK10 = np.array([0, 1, 2, 3, 4, 6, 8, 10, 0, -1, -2, -3, -4, -6, -8, -10], dtype=np.int64)


def scale_bytes_per_block(layout: int) -> int:
    """Number of scale bytes after ``qs`` ("Block Layout": e[2] dual, e fast)."""
    if layout == DUAL:
        return 2
    if layout == FAST:
        return 1
    raise ValueError(f"unknown layout {layout}")


def block_bytes(layout: int) -> int:
    """Bytes per 32-weight block: 16 bytes of indices plus the scale bytes."""
    return QS_BYTES + scale_bytes_per_block(layout)


def bits_per_weight(layout: int) -> float:
    return 8.0 * block_bytes(layout) / WEIGHTS_PER_BLOCK


def row_bytes(layout: int, k: int) -> int:
    """Bytes of one matrix row under reading R-ROW (K/32 blocks back to back)."""
    if k % WEIGHTS_PER_BLOCK:
        raise ValueError("k must be a multiple of 32")
    return (k // WEIGHTS_PER_BLOCK) * block_bytes(layout)


def e4m3_value(u):
    """Textbook E4M3 magnitude of the 7-bit field ``u`` (exponent bias 7).

    exponent field e = u >> 3, mantissa m = u & 7:
      e >= 1: 2**(e - 7) * (1 + m / 8)
      e == 0: m * 2**-9                (reading R-SUB)
    The all-ones pattern is not special-cased (reading R-NAN): it gives 480.
    """
    u = np.asarray(u, dtype=np.int64)
    e = u >> 3
    m = u & 7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = m * 2.0 ** -9
    return np.where(e == 0, sub, normal)


def scale_value(b):
    """Decoded half-scale of a scale byte ("Scale Format"; readings R-HALF, R-SIGN)."""
    b = np.asarray(b, dtype=np.int64)
    return 0.5 * e4m3_value(b & 0x7F)


def split_blocks(w: np.ndarray, layout: int, n: int, k: int):
    """View packed bytes as blocks and return (qs, e).

    qs: uint8 (n, k/32, 16); e: uint8 (n, k/32, 1 or 2). Field order follows the
    struct members in "Block Layout" (qs first, then the scale byte(s)).
    """
    nb = k // WEIGHTS_PER_BLOCK
    bb = block_bytes(layout)
    blocks = np.ascontiguousarray(w, dtype=np.uint8).reshape(n, nb, bb)
    return blocks[:, :, :QS_BYTES], blocks[:, :, QS_BYTES:]


def nibble_indices(qs: np.ndarray) -> np.ndarray:
    """32 codebook indices per block under reading R-NIB (low plane, then high plane)."""
    lo = qs & 0x0F
    hi = qs >> 4
    return np.concatenate([lo, hi], axis=-1).astype(np.int64)


def per_weight_scale(e: np.ndarray, layout: int) -> np.ndarray:
    """Scale of each of the 32 weights of every block.

    Dual ("one per 16-weight half"): weights 0..15 use e[0], 16..31 use e[1].
    Fast ("one ... scale for the whole block"): all 32 use e.
    """
    s = scale_value(e)
    if layout == DUAL:
        return np.repeat(s, 16, axis=-1)
    return np.repeat(s, 32, axis=-1)


def dequantize(w: np.ndarray, layout: int, n: int, k: int) -> np.ndarray:
    """Real value of every weight, fp64, shape (n, k): codebook[idx] * S (reading R-ZERO)."""
    qs, e = split_blocks(w, layout, n, k)
    codes = CODEBOOK10[nibble_indices(qs)].astype(np.float64)
    vals = codes * per_weight_scale(e, layout)
    return vals.reshape(n, k)


def dequantize_f32(w: np.ndarray, layout: int, n: int, k: int) -> np.ndarray:
    """Dequantized weights as fp32. Every codebook value times every decoded scale is
    exactly representable in fp32, so this cast is exact."""
    return dequantize(w, layout, n, k).astype(np.float32)


def gemv(w: np.ndarray, layout: int, n: int, k: int, x: np.ndarray):
    """Decode matvec y[b, r] = sum_c W[r, c] * x[b, c], exact in fp64.

    The page names gemv as the decode hot path ("Kernel System"; "Integration
    Options", Option 2). ``x`` is (batch, k) fp64 (already exact copies of the
    fp16/bf16 activations). Returns (y, den) where den = sum_c |W[r, c] * x[b, c]| is
    the denominator of the normalized error.
    """
    wd = dequantize(w, layout, n, k)
    x = np.asarray(x, dtype=np.float64).reshape(-1, k)
    y = x @ wd.T
    den = np.abs(x) @ np.abs(wd).T
    return y, den


def gemv_rows(w: np.ndarray, layout: int, n: int, k: int, x: np.ndarray, rows: np.ndarray):
    """``gemv`` restricted to the given row indices (for sampled checks at full size)."""
    rb = row_bytes(layout, k)
    wr = np.ascontiguousarray(np.asarray(w, dtype=np.uint8).reshape(n, rb)[rows])
    return gemv(wr, layout, len(rows), k, x)


def gemm(w: np.ndarray, layout: int, n: int, k: int, a: np.ndarray):
    """Prefill product C[m, r] = sum_c A[m, c] * W[r, c] (C = A W^T), exact in fp64.

    The page names a weight-only 4-bit GEMM for prefill ("Kernel System",
    w4a16_gemm). Returns (C, den) with den = |A| |W|^T.
    """
    wd = dequantize(w, layout, n, k)
    a = np.asarray(a, dtype=np.float64)
    return a @ wd.T, np.abs(a) @ np.abs(wd).T


def gemm_rows(w: np.ndarray, layout: int, n: int, k: int, a: np.ndarray, cols: np.ndarray):
    """``gemm`` restricted to the given weight rows (= output columns of C)."""
    rb = row_bytes(layout, k)
    wr = np.ascontiguousarray(np.asarray(w, dtype=np.uint8).reshape(n, rb)[cols])
    return gemm(wr, layout, len(cols), k, a)


# ------------------------------------------------------------------ quantizer
# The page defines the value a block decodes to but no encoder; of encoding it says only
# that the largest magnitude was retuned from 12 to 10 to limit the pull of outliers
# ("Codebook10 Value Table"). Reading R-QUANT, the plainest encoder the decoder supports:
#   * a group (a 16-weight half for dual, the whole block for fast) takes the smallest
#     finite half-scale S(b), b in 0..126 (bit 7 clear; 0x7F is non-finite), with
#     10 * S(b) >= max |w| over the group, saturating at b = 126 (S = 224);
#   * each weight takes the codebook entry nearest to w / S: its magnitude index is the
#     number of midpoints m of consecutive magnitudes with |w| > m * S (a tie goes to the
#     smaller magnitude), and its sign bit is set when w < 0 and the magnitude is not 0
#     (a zero, of either sign, is index 0).
# Every 10 * S(b) and m * S(b) is exact in fp32 and fp64, so no rounding decides a code
# and any implementation that compares exactly gets the same bytes.
MAX_FINITE_SCALE_BYTE = 126
MIDPOINTS = (0.5, 1.5, 2.5, 3.5, 5.0, 7.0, 9.0)  # between 0,1,2,3,4,6,8,10


def quantize(v, layout: int) -> np.ndarray:
    """Encode real weights (n, k), k % 32 == 0, to packed blocks (n, row_bytes) (R-QUANT).

    Inputs are used exactly (fp16/bf16/fp32 all convert exactly to fp64); non-finite
    inputs give unspecified bytes."""
    v = np.asarray(v, dtype=np.float64)
    n, k = v.shape
    if k % WEIGHTS_PER_BLOCK:
        raise ValueError("k must be a multiple of 32")
    nb = k // WEIGHTS_PER_BLOCK
    group = 16 if layout == DUAL else 32
    g = v.reshape(n, nb, WEIGHTS_PER_BLOCK // group, group)
    amax = np.abs(g).max(axis=-1)
    reach = 10.0 * scale_value(np.arange(MAX_FINITE_SCALE_BYTE + 1))  # strictly increasing
    b = np.minimum(np.searchsorted(reach, amax, side="left"), MAX_FINITE_SCALE_BYTE)
    s = scale_value(b)[..., None]
    mag = np.zeros(g.shape, dtype=np.int64)
    for m in MIDPOINTS:
        mag += np.abs(g) > m * s
    idx = (mag + 8 * ((g < 0) & (mag > 0))).reshape(n, nb, WEIGHTS_PER_BLOCK)
    qs = (idx[..., :16] | (idx[..., 16:] << 4)).astype(np.uint8)  # R-NIB
    e = b.astype(np.uint8).reshape(n, nb, scale_bytes_per_block(layout))
    return np.concatenate([qs, e], axis=-1).reshape(n, nb * block_bytes(layout))


def validate(w: np.ndarray, layout: int, n: int, k: int):
    """Row validation ("Scale Format"): a tensor is accepted iff no scale byte is
    non-finite as E4M3, i.e. no byte has its low seven bits all set.

    Returns (ok, first_bad_block) with blocks numbered row-major (row * K/32 + j);
    first_bad_block is -1 when ok.
    """
    _, e = split_blocks(w, layout, n, k)
    bad = np.any((e & 0x7F) == 0x7F, axis=-1).reshape(-1)
    idx = np.flatnonzero(bad)
    if idx.size == 0:
        return True, -1
    return False, int(idx[0])


def normalized_error(y, y_ref, den) -> float:
    """max |y - y_ref| / den over all outputs; where den == 0 the output must be exactly
    zero (otherwise the error is infinite)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    diff = np.abs(y - y_ref)
    zero = den == 0
    if np.any(zero & (diff != 0)):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(diff[~zero] / den[~zero]))
