"""Seeded synthetic inputs for the ROCmFP4 contraction.

Shared by the tests, the benchmark and the oracle checks. This package only draws
random bytes and random activations and lays them out in the block byte order of
"Feasibility Report: Porting ROCmFP4 to Atlas", "Block Layout" (16 index bytes, then
the scale byte(s)); it decodes nothing and holds none of the method's arithmetic.

Recipe (every workload, seed fixed per workload):

* index bytes: uniform 0..255, so both 4-bit indices of a byte are uniform 0..15;
* scale bytes: (E << 3) | M with exponent field E uniform in 4..9 and mantissa M
  uniform in 0..7, bit 7 clear (finite, unsigned E4M3); or, for the scale-range
  tests, uniform over all 254 finite bytes (every byte but 0x7F and 0xFF: bit 7 set
  or clear, exponent field 0 included), with the first 254 scale bytes of each half
  running through all of them in a seeded random order;
* stress blocks (down-projection workload): a fraction of the blocks, drawn without
  replacement, get every index in {7, 15} (magnitude 10, random sign) and scale
  (15 << 3) | M with M uniform in 0..6 (the largest finite exponent);
* activations: standard normal float32, rounded to nearest even into fp16 (NumPy) or
  bf16 (torch);
* real-valued weights (quantizer input): standard normal times a per-row scale
  0.02 * exp(N(0, 0.5^2)), with 0.1 % of the entries (drawn without replacement)
  multiplied by 20 as outliers, in float32, then rounded to nearest even into bf16
  or fp16 where asked.

Draw order per workload: index bytes, scale bytes, stress choice, activations.
"""

from __future__ import annotations

import numpy as np

DUAL = 0
FAST = 1
_BLOCK_BYTES = {DUAL: 18, FAST: 17}
_SCALES = {DUAL: 2, FAST: 1}


def block_bytes(layout: int) -> int:
    return _BLOCK_BYTES[layout]


def row_bytes(layout: int, k: int) -> int:
    assert k % 32 == 0
    return (k // 32) * _BLOCK_BYTES[layout]


# The 254 byte values a validated row may hold as a scale byte ("Scale Format": the
# bytes whose low seven bits are all ones are the non-finite ones).
FINITE_SCALE_BYTES = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)


def weights(rng: np.random.Generator, layout: int, n: int, k: int,
            stress_frac: float = 0.0, exp_lo: int = 4, exp_hi: int = 9,
            all_scales: bool = False) -> np.ndarray:
    """Packed weight bytes, uint8 array of shape (n, row_bytes). With all_scales, the
    scale bytes are drawn from every finite byte (see the module recipe)."""
    nb = k // 32
    ns = _SCALES[layout]
    qs = rng.integers(0, 256, size=(n, nb, 16), dtype=np.uint8)
    if all_scales:
        sc = FINITE_SCALE_BYTES[rng.integers(0, FINITE_SCALE_BYTES.size, size=(n, nb, ns))]
        first = min(n * nb, FINITE_SCALE_BYTES.size)
        for h in range(ns):
            sc.reshape(n * nb, ns)[:first, h] = rng.permutation(FINITE_SCALE_BYTES)[:first]
    else:
        ex = rng.integers(exp_lo, exp_hi + 1, size=(n, nb, ns), dtype=np.uint8)
        mu = rng.integers(0, 8, size=(n, nb, ns), dtype=np.uint8)
        sc = (ex << 3) | mu
    if stress_frac > 0.0:
        total = n * nb
        cnt = int(np.floor(stress_frac * total))
        pick = rng.choice(total, size=cnt, replace=False)
        lo = np.where(rng.integers(0, 2, size=(cnt, 16), dtype=np.uint8) == 1, 15, 7).astype(np.uint8)
        hi = np.where(rng.integers(0, 2, size=(cnt, 16), dtype=np.uint8) == 1, 15, 7).astype(np.uint8)
        qs.reshape(total, 16)[pick] = lo | (hi << 4)
        smu = rng.integers(0, 7, size=(cnt, ns), dtype=np.uint8)
        sc.reshape(total, ns)[pick] = (15 << 3) | smu
    blocks = np.concatenate([qs, sc], axis=2)
    return np.ascontiguousarray(blocks.reshape(n, nb * _BLOCK_BYTES[layout]))


def activations(rng: np.random.Generator, rows: int, k: int, dtype: str):
    """(rows, k) activations as a CPU torch tensor of dtype 'f16' or 'bf16'."""
    import torch

    x = rng.standard_normal(size=(rows, k), dtype=np.float32)
    if dtype == "f16":
        return torch.from_numpy(x.astype(np.float16))
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16)
    raise ValueError(dtype)


def real_weights(rng: np.random.Generator, n: int, k: int, dtype: str):
    """(n, k) real-valued weights as a CPU torch tensor of dtype 'f32', 'bf16' or 'f16'."""
    import torch

    row = 0.02 * np.exp(0.5 * rng.standard_normal(size=(n, 1), dtype=np.float32))
    v = rng.standard_normal(size=(n, k), dtype=np.float32) * row.astype(np.float32)
    pick = rng.choice(n * k, size=(n * k) // 1000, replace=False)
    v.reshape(-1)[pick] *= np.float32(20.0)
    t = torch.from_numpy(v)
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f16":
        return t.to(torch.float16)
    raise ValueError(dtype)


def weights_device(layout: int, n: int, k: int, seed: int, device):
    """Same distribution as ``weights`` (no stress), drawn on the device with a torch
    generator; used for large resident sets (rotation copies, the 64-layer sweep)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    nb = k // 32
    ns = _SCALES[layout]
    qs = torch.randint(0, 256, (n, nb, 16), generator=g, device=device, dtype=torch.uint8)
    ex = torch.randint(4, 10, (n, nb, ns), generator=g, device=device, dtype=torch.uint8)
    mu = torch.randint(0, 8, (n, nb, ns), generator=g, device=device, dtype=torch.uint8)
    sc = (ex << 3) | mu
    return torch.cat([qs, sc], dim=2).reshape(n, nb * _BLOCK_BYTES[layout]).contiguous()


def activations_device(rows: int, k: int, dtype: str, seed: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((rows, k), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.float16 if dtype == "f16" else torch.bfloat16)


# The five workloads. Shapes: n = weight rows (outputs), k = reduction length.
CONFIGS = {
    "tiny": dict(layout=DUAL, n=256, k=512, xdtype="f16", batch=1, stress=0.0, seed=0),
    "up": dict(layout=DUAL, n=17408, k=5120, xdtype="f16", batch=1, stress=0.0, seed=0),
    "down": dict(layout=FAST, n=5120, k=17408, xdtype="bf16", batch=8, stress=0.01, seed=0),
    "prefill": dict(layout=DUAL, n=17408, k=5120, m=2048, seed=0),
}

# Decode sweep of a 27B-class dense decoder: 64 layers, 7 projections, all dual.
SWEEP_LAYERS = 64
SWEEP_SHAPES = [  # (name, n, k)
    ("q", 6144, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 6144),
    ("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408),
]


def gemv_inputs(name: str, batch: int | None = None):
    """(w_bytes uint8 (n, row_bytes), x torch CPU (batch, k), cfg) for a GEMV workload."""
    cfg = dict(CONFIGS[name])
    rng = np.random.default_rng(cfg["seed"])
    w = weights(rng, cfg["layout"], cfg["n"], cfg["k"], cfg["stress"])
    b = cfg["batch"] if batch is None else batch
    x_all = activations(rng, cfg["batch"], cfg["k"], cfg["xdtype"])
    x = x_all[:b].contiguous()
    cfg["batch"] = b
    return w, x, cfg


def gemm_inputs(name: str = "prefill"):
    cfg = dict(CONFIGS[name])
    rng = np.random.default_rng(cfg["seed"])
    w = weights(rng, cfg["layout"], cfg["n"], cfg["k"])
    a = activations(rng, cfg["m"], cfg["k"], "bf16")
    return w, a, cfg
