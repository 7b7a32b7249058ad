"""CPU oracle for the ROCmFP4 contraction -- test infrastructure only.

Importable from tests/, ``__graft_entry__.smoke()`` and bench.py's CPU-baseline leg;
never from the product package.
"""

from .rfp4_oracle import *  # noqa: F401,F403
from .rfp4_oracle import (  # noqa: F401
    CODEBOOK10,
    DUAL,
    FAST,
    bits_per_weight,
    block_bytes,
    dequantize,
    dequantize_f32,
    e4m3_value,
    gemm,
    gemm_rows,
    gemv,
    gemv_rows,
    nibble_indices,
    normalized_error,
    quantize,
    row_bytes,
    scale_value,
    split_blocks,
    validate,
)
