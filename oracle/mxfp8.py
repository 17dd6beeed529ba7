"""MXFP8 block-scaled projection, plain fp64 CPU statement (test infrastructure only).

The pages carry MXFP8 weights as a card format, E4M3 elements in blocks of 32
with one E8M0 scale a block, run as a gemv and as a wide prompt GEMM with an
fp32 tile [FP4-Local checkpoints on DGX Spark, §4 Round 1, #521].

Readings: the weight is [N, K] (output-major), a block is 32 consecutive K
elements of one output row; activations stay bfloat16 (the pages' W8A8 variant,
#769, quantizes them and is a separate path); y = x . W^T accumulated exactly
here and rounded once to bfloat16.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .moe import OracleRefusal


def validate(x_bits, w, s, M, N, K):
    if min(M, N, K) < 1 or K % 32:
        raise OracleRefusal("shape: M, N, K >= 1 and K % 32 == 0")
    if x_bits.shape != (M, K) or w.shape != (N, K) or s.shape != (N, K // 32):
        raise OracleRefusal("shape: x, w or s")
    if np.any((w & 0x7F) == 0x7F):
        raise OracleRefusal("NaN E4M3 code in the weight")
    if np.any(s == 0xFF):
        raise OracleRefusal("NaN E8M0 scale")


def dequant_mxfp8(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W[n, i] = E4M3(w[n, i]) * 2^(s[n, i // 32] - 127), fp64 [N, K] (exact)."""
    return F.E4M3_TABLE[w] * np.repeat(F.E8M0_TABLE[s], 32, axis=-1)


def mxfp8_gemm(x_bits, w, s, rows=None, cols=None):
    """y = x . W^T (fp64) and out = bf16_rne(y); optionally only for a subset
    of rows of x and columns of W. Returns (y, out_bits, mass) where
    mass = |x| . |W|^T is the L1 mass of each output's contraction."""
    M, K = x_bits.shape
    N = w.shape[0]
    validate(x_bits, w, s, M, N, K)
    if rows is not None:
        x_bits = x_bits[np.asarray(rows)]
    if cols is not None:
        w = w[np.asarray(cols)]
        s = s[np.asarray(cols)]
    X = F.bf16_bits_to_f64(x_bits)
    W = dequant_mxfp8(w, s)
    y = X @ W.T
    mass = np.abs(X) @ np.abs(W).T
    return y, F.bf16_rne_bits(y), mass
