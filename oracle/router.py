"""Router projection, plain fp64 CPU statement (test infrastructure only).

Only tests/, the package's smoke check and the benchmark's CPU-baseline leg use
this module; the GPU path never imports it.

The router logits are the token activations times the router matrix, the matrix
kept in its stored BF16 words rather than widened [FP4-Local checkpoints on DGX
Spark, §4 Round 1, #732], summed on a float32 tile [same page, §4 Round 1, #763]:

    logits[t, e] = sum_i x[t, i] * W_r[e, i]

with x bfloat16 [T, d] and W_r bfloat16 [E, d]. Every product of two bfloat16
values is exact in fp64 (8 + 8 significant bits); the sum over i is taken in fp64,
whose own rounding (at most d * 2^-53 of the mass below) is far under the float32
tolerance the GPU is held to.

Float32 tolerance (derived, not from the pages): a sum of n terms in float32, in
any order and grouping, differs from the exact sum by at most (n - 1) * u *
sum |terms| (u = 2^-24, first order); with the d products, at most 8 further
additions of partial sums and the final rounding, the bound used is
(d + 8) * u * mass, where mass[t, e] = sum_i |x[t, i] * W_r[e, i]|.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

U32 = 2.0 ** -24  # float32 unit roundoff


def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray, rows=None):
    """Exact router logits and their mass.

    x_bits uint16 [T, d] and wr_bits uint16 [E, d] are bfloat16 bits. ``rows``
    (optional) selects token rows. Returns (logits float64 [t, E], mass float64
    [t, E])."""
    x = F.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    w = F.bf16_bits_to_f64(np.asarray(wr_bits, dtype=np.uint16))
    if x.shape[1] != w.shape[1]:
        raise ValueError("shape: x and W_r must have the same row length d")
    if rows is not None:
        x = x[np.asarray(rows)]
    return x @ w.T, np.abs(x) @ np.abs(w).T


def router_tolerance(d: int, mass: np.ndarray) -> np.ndarray:
    """Largest |float32 result - exact| any summation order may produce."""
    return (d + 8) * U32 * mass
