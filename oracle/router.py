"""Router projection and routing policies, plain fp64 CPU statement (test
infrastructure only).

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

Routing policies. The pages make the router's normalization policy a named value
[bloomery 0.3.9 release notes, From our contributors, #772] without listing the
values; the readings taken here (each listed in the design notes):

  0 SOFTMAX_RENORM  softmax over the experts, keep the top k, renormalize over
                    them (= softmax over the k selected logits); the default;
  1 SOFTMAX         the same top k, weights = the softmax over all E experts,
                    not renormalized (they sum to at most 1);
  2 SIGMOID_RENORM  weights = sigmoid of each selected logit, divided by their sum;
  3 SIGMOID         weights = sigmoid of each selected logit, as is.

Every policy selects the same way: the k largest selection keys, ties to the
lower expert index, in that order. The key is the logit, or with a correction
bias b (one float32 an expert) the float32 sum logit + b[e], rounded to float32
as the GPU adds it -- the bias moves the choice only; the weights always use the
unbiased logits. Softmax and sigmoid are monotone, so without a bias the choice
is the same under every policy.
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


SOFTMAX_RENORM, SOFTMAX, SIGMOID_RENORM, SIGMOID = 0, 1, 2, 3


def selection_keys(logits: np.ndarray, bias=None) -> np.ndarray:
    """float32 keys: the logits, or the float32-rounded sums logit + bias[e]."""
    lg = np.asarray(logits, dtype=np.float32)
    if bias is None:
        return lg
    return (lg + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)


def route_policy(logits: np.ndarray, k: int, policy: int = SOFTMAX_RENORM, bias=None):
    """Top-k choice and weights under a routing policy (see the module docstring).

    Returns ids int32 [T, k] (selection order) and w float64 [T, k]."""
    if policy not in (SOFTMAX_RENORM, SOFTMAX, SIGMOID_RENORM, SIGMOID):
        raise ValueError(f"unknown routing policy {policy}")
    keys = selection_keys(logits, bias).astype(np.float64)
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # primary: key descending (-0.0 == +0.0), secondary: expert index ascending
        ids[t] = np.lexsort((np.arange(E), -keys[t]))[:k]
    sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1)
    if policy == SOFTMAX_RENORM:
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        w = ex / ex.sum(axis=1, keepdims=True)
    elif policy == SOFTMAX:
        m = lg.max(axis=1, keepdims=True)
        w = np.exp(sel - m) / np.exp(lg - m).sum(axis=1, keepdims=True)
    else:
        sg = np.where(sel >= 0, 1.0 / (1.0 + np.exp(-np.abs(sel))), np.exp(-np.abs(sel)) / (1.0 + np.exp(-np.abs(sel))))
        w = sg / sg.sum(axis=1, keepdims=True) if policy == SIGMOID_RENORM else sg
    return ids, w
