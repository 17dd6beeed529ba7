"""MXFP8 activations and the W8A8 MXFP8 projection, plain fp64 CPU statement (test
infrastructure only).

Only tests/, the package's smoke check and the benchmark's CPU-baseline leg use this
module; the GPU path never imports it.

The pages run an MXFP8 projection with 8-bit activations (W8A8) beside the bf16-activation
one [FP4-Local checkpoints on DGX Spark, §4 Round 1, #769; "Weight and activation formats
on the GB10 tensor cores"], and count such variants apart from the exact path since they
change results. The activation format is MXFP8 as the weights: E4M3 elements in blocks
of 32 along K with one E8M0 scale a block. The conversion follows the OCP Microscaling
Formats (MX) v1.0 specification, in the order it gives:

1. per block of 32 values v_i, the shared exponent is floor(log2(max_i |v_i|)) minus the
   element format's largest exponent (8 for E4M3, whose largest value is 1.75 * 2^8);
   the block scale is 2^shared_exp, as an E8M0 code (exponent + 127), clamped to the
   code range 0 .. 254;
2. each element is v_i / scale rounded to the nearest E4M3 value, ties to even.

Readings taken where the specification leaves the choice to the implementation (listed
in the design notes):

* overflow: v_i / scale lies in [256, 512) for the block's largest magnitude, past the
  E4M3 maximum 448; such values saturate to +-448 (the specification allows saturating
  or NaN; a NaN would poison the product);
* an all-zero block (log2 0 undefined) gets code 0 (2^-127) and zero elements;
* E4M3 subnormals (multiples of 2^-9 below 2^-6) are kept, and a value that rounds to
  zero keeps its sign (-0 is the code 0x80; both zero codes are the value 0).

The projection is then y = x_hat . W^T with x_hat[m, i] = E4M3(xq[m, i]) *
2^(xs[m, i / 32] - 127) and W as in oracle/mxfp8.py, in exact fp64 arithmetic of those
values, and out = bf16_rne(y).
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .moe import OracleRefusal
from . import mxfp8

E4M3_EMAX = 8          # largest exponent of an E4M3 value (448 = 1.75 * 2^8)
E4M3_MAX = 448.0

# the 127 non-negative finite E4M3 values by code (0x00 .. 0x7E), increasing
_POS_VALUES = F.E4M3_TABLE[:127]


def e4m3_rne_sat(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each float64 value, ties to the even code (an even mantissa
    field; the codes are in increasing value order, so the even code is the even index),
    magnitudes above 448 saturated to 448; returns uint8 codes (sign in bit 7)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS_VALUES[hi], hi, code)           # exact values
    sign = np.signbit(v).astype(np.uint8) << 7  # the sign is kept, zero results included (-0 is 0x80)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_mx(x_bits: np.ndarray):
    """bf16 activations [M, K] (bits) -> (codes uint8 [M, K], scales uint8 [M, K/32])."""
    x = F.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    M, K = x.shape
    if K % 32:
        raise OracleRefusal("shape: K % 32 != 0")
    if not np.all(np.isfinite(x)):
        raise OracleRefusal("non-finite activation")
    blocks = x.reshape(M, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))           # amax = m 2^e, m in [0.5, 1)
    shared = (e - 1) - E4M3_EMAX                               # floor(log2 amax) - emax
    code = np.clip(shared + 127, 0, 254)
    code = np.where(amax > 0, code, 0).astype(np.uint8)
    scale = np.ldexp(1.0, code.astype(np.int64) - 127)
    q = e4m3_rne_sat(blocks / scale[:, :, None])
    return q.reshape(M, K), code


def dequant_mx(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 codes [.., K] and E8M0 scales [.., K/32] -> fp64 values (exact)."""
    return F.E4M3_TABLE[codes] * np.repeat(F.E8M0_TABLE[scales], 32, axis=-1)


def mxfp8_gemm_mx(xq, xs, w, s, rows=None, cols=None):
    """y = x_hat . W^T (fp64) with MXFP8 activations and weights; returns (y, out_bits,
    mass), mass = |x_hat| . |W|^T; optionally a subset of rows / weight rows."""
    M, K = xq.shape
    N = w.shape[0]
    mxfp8.validate(np.zeros((M, K), np.uint16), w, s, M, N, K)
    if np.any((xq & 0x7F) == 0x7F) or np.any(xs == 0xFF):
        raise OracleRefusal("NaN code in the MXFP8 activations")
    if rows is not None:
        xq, xs = xq[np.asarray(rows)], xs[np.asarray(rows)]
    if cols is not None:
        w, s = w[np.asarray(cols)], s[np.asarray(cols)]
    X = dequant_mx(xq, xs)
    W = mxfp8.dequant_mxfp8(w, s)
    y = X @ W.T
    return y, F.bf16_rne_bits(y), np.abs(X) @ np.abs(W).T
