"""Routed NVFP4 mixture-of-experts FFN, plain fp64 CPU statement (test infrastructure only).

The layer, as the pages describe it: a whole batch of tokens is routed in one
run so every selected expert is read once for all its rows [FP4-Local
checkpoints on DGX Spark, §4 Round 1, #740 and #808]; each routed NVFP4 expert
is a gate, an up and a down product over weights held in their stored bytes,
with a scale per expert [same page, §4 Round 1, #489, #517, #545]; gate, up and
SwiGLU form one step [same page, §4 Round 1, #766]; the down rows are formed by
rounding to nearest even and widened in the sum [same page, §4 remaining items,
#914]; the expert rows are summed in the combine [same page, §4 Round 1, #701];
the router weights are normalized under a named policy [bloomery 0.3.9 release
notes, From our contributors / Fixed, #772].

Readings taken where the pages are silent (each is listed in the design notes):

1. Router policy: softmax over the experts, keep the top k, renormalize to sum
   one -- equal to a softmax over the k selected logits.
2. Selection is on the raw float32 logits, ordered by (logit descending, expert
   index ascending); -0.0 equals +0.0. The output order is that order.
3. Row lists: a stable counting sort of the flat assignments a = t*k + j by
   expert; row_of is its inverse.
4. Dequantization: W[n, i] = E2M1(code) * E4M3(scale[n, i // 16]), exact; the
   per-expert fp32 tensor scale multiplies the product's accumulator. There is
   one tensor scale per expert and projection (gate, up, down); the pages'
   single scale per expert is the case of three equal values.
5. Activations stay bfloat16 (no activation quantization, input scales ignored,
   [same page, §9 Rules and related work, Accuracy]).
6. h = bf16_rne(silu(G) * U), rounded once, directly from the exact value.
7. The down rows are kept unrounded (fp64 here, fp32 on the GPU); the combine
   rounds once to bfloat16 at the end.
8. SwiGLU is silu on the gate branch times the up branch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import formats as F


class OracleRefusal(ValueError):
    """An input the oracle refuses by name (non-finite, NaN codes, bad shapes)."""


# ----------------------------------------------------------------------------- validation
def validate_moe(T, d, f, E, k, x, logits, experts=None):
    """Refuse bad inputs by name: the pages refuse structural errors by name
    [FP4-Local checkpoints on DGX Spark, §9 Rules and related work, Accuracy]
    and refuse non-finite values [same page, §10, #597 and #710]."""
    if min(T, d, f, E, k) < 1:
        raise OracleRefusal("shape: T, d, f, E, k must be >= 1")
    if k > E:
        raise OracleRefusal("shape: k > E")
    if d % 32 or f % 32:
        raise OracleRefusal("shape: d and f must be multiples of 32")
    if x.shape != (T, d) or logits.shape != (T, E):
        raise OracleRefusal("shape: x or logits")
    if not np.all(np.isfinite(logits)):
        raise OracleRefusal("non-finite router logit")
    if experts is not None:
        for nm in ("gate_s", "up_s", "down_s"):
            s = experts[nm]
            if np.any((s & 0x7F) == 0x7F):
                raise OracleRefusal(f"NaN E4M3 code in {nm}")
        for nm in ("gate_ts", "up_ts", "down_ts"):
            if not np.all(np.isfinite(experts[nm])):
                raise OracleRefusal(f"non-finite tensor scale {nm}")


# ----------------------------------------------------------------------------- routing
def route(logits: np.ndarray, k: int):
    """Top-k routing with renormalized softmax weights.

    Per token t: order the experts by (logit descending, index ascending) and
    keep the first k; w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) in fp64,
    where l_0 is the largest selected logit.

    Returns ids int32 [T, k] and w float64 [T, k].
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    vals = logits.astype(np.float64)
    idx = np.broadcast_to(np.arange(E), (T, E))
    # np.lexsort sorts by the last key first: primary -value, secondary index.
    # -(-0.0) == 0.0 compares equal to 0.0, so signed zeros tie and fall to the index.
    order = np.empty((T, E), dtype=np.int64)
    for t in range(T):
        order[t] = np.lexsort((idx[t], -vals[t]))
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(vals, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


@dataclass
class RowLists:
    counts: np.ndarray       # int32 [E]
    offsets: np.ndarray      # int32 [E+1], exclusive prefix sum, offsets[E] = T*k
    sorted_rows: np.ndarray  # int32 [T*k], assignment ids grouped by expert, increasing inside
    row_of: np.ndarray       # int32 [T*k], inverse: row_of[sorted_rows[p]] = p


def row_lists(ids: np.ndarray, E: int) -> RowLists:
    """Stable counting sort of the assignments by expert (one list per expert)."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.argsort(flat, kind="stable")
    row_of = np.empty_like(sorted_rows)
    row_of[sorted_rows] = np.arange(flat.size)
    return RowLists(counts.astype(np.int32), offsets.astype(np.int32),
                    sorted_rows.astype(np.int32), row_of.astype(np.int32))


# ----------------------------------------------------------------------------- dequantization
def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[n, i] = E2M1(nibble i of row n) * E4M3(scales[n, i // 16]), fp64 [N, K].

    Exact: an E2M1 significand has at most 2 bits and an E4M3 one at most 4, so
    every product has at most 6 significant bits (and is exact in bfloat16 too).
    """
    vals = F.unpack_e2m1(codes)                        # [N, K]
    sc = F.E4M3_TABLE[np.asarray(scales, dtype=np.uint8)]  # [N, K/16]
    return vals * np.repeat(sc, 16, axis=-1)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)), evaluated without overflow on either side."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    eg = np.exp(g[~pos])
    out[~pos] = g[~pos] * eg / (1.0 + eg)
    return out


def experts_dict(inp) -> dict:
    return {nm: getattr(inp, nm) for nm in
            ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")}


@dataclass
class FFNResult:
    rows: np.ndarray        # row-list positions p computed (int64)
    y_rows: np.ndarray      # float64 [len(rows), d]: ts_d * (H @ W_d^T), unrounded
    h_bits: np.ndarray      # uint16 [len(rows), f]: H = bf16_rne(silu(G) * U)
    mass_y: np.ndarray      # float64 [len(rows), d]: |ts_d| * (|H| @ |W_d|^T)
    slack_h: np.ndarray     # float64 [len(rows), d]: 1-ulp flips of ambiguous h elements


# 2^-20: relative size of the fp32 accumulation differences the slack allows for
ACC_REL = 2.0 ** -20


def expert_ffn(x_bits, T, d, f, E, k, experts: dict, rl: RowLists, rows=None, map_fn=map) -> FFNResult:
    """Per routed row p (row-list order): with t = sorted_rows[p] // k and the
    expert e owning p,

        G = ts_g[e] * (x[t] . W_g[e]^T),  U = ts_u[e] * (x[t] . W_u[e]^T)
        H = bf16_rne(silu(G) * U)
        O = ts_d[e] * (H . W_d[e]^T)      (kept unrounded)

    ``rows`` restricts the computation to a subset of row-list positions (every
    row is independent of the others), for sampled checks at large sizes.
    Experts are independent too: ``map_fn`` (default the builtin map; e.g. a
    thread pool's map) applies the per-expert computation to the list of experts,
    which changes nothing in the arithmetic.
    Also returns the slack terms used by the acceptance rule (see band.py).
    """
    offsets = rl.offsets.astype(np.int64)
    if rows is None:
        rows = np.arange(T * k, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.size
    y_rows = np.zeros((n, d))
    mass_y = np.zeros((n, d))
    slack_h = np.zeros((n, d))
    h_bits = np.zeros((n, f), dtype=np.uint16)
    owner = np.searchsorted(offsets, rows, side="right") - 1   # expert of each row

    def one_expert(e):
        sel = np.nonzero(owner == e)[0]
        p = rows[sel]
        tok = rl.sorted_rows[p].astype(np.int64) // k
        X = F.bf16_bits_to_f64(x_bits[tok])                    # [n_e, d]
        Wg = dequant_nvfp4(experts["gate_q"][e], experts["gate_s"][e])   # [f, d]
        Wu = dequant_nvfp4(experts["up_q"][e], experts["up_s"][e])
        Wd = dequant_nvfp4(experts["down_q"][e], experts["down_s"][e])   # [d, f]
        tg = float(experts["gate_ts"][e])
        tu = float(experts["up_ts"][e])
        td = float(experts["down_ts"][e])
        G = tg * (X @ Wg.T)
        U = tu * (X @ Wu.T)
        sg = silu(G)
        h_exact = sg * U
        H = F.bf16_rne(h_exact)
        O = td * (H @ Wd.T)
        hb = F.bf16_rne_bits(h_exact)
        # ---- slack terms
        # L1 masses: every factor taken by magnitude (tensor scales can be negative)
        aX = np.abs(X)
        mass_g = abs(tg) * (aX @ np.abs(Wg).T)
        mass_u = abs(tu) * (aX @ np.abs(Wu).T)
        # d silu / dg = s(g) * (1 + g * (1 - s(g))), s = logistic; h = silu(g) * u
        sig = np.where(G >= 0, 1.0 / (1.0 + np.exp(-np.abs(G))), np.exp(-np.abs(G)) / (1.0 + np.exp(-np.abs(G))))
        dsilu = sig * (1.0 + G * (1.0 - sig))
        dh = np.abs(dsilu * U) * ACC_REL * mass_g + np.abs(sg) * ACC_REL * mass_u + ACC_REL * np.abs(h_exact)
        ulp = F.bf16_ulp(H)
        # an element is ambiguous when a bfloat16 rounding boundary (a midpoint
        # between neighbours) lies inside h_exact +- dh
        lo_mid = H - ulp / 2.0
        hi_mid = H + ulp / 2.0
        amb = (h_exact - dh <= lo_mid) | (h_exact + dh >= hi_mid)
        aWd = np.abs(Wd)
        my = abs(td) * (np.abs(H) @ aWd.T)
        sh = abs(td) * ((amb * ulp) @ aWd.T)
        return sel, O, hb, my, sh

    for sel, O, hb, my, sh in map_fn(one_expert, list(np.unique(owner))):
        y_rows[sel] = O
        h_bits[sel] = hb
        mass_y[sel] = my
        slack_h[sel] = sh
    return FFNResult(rows=rows, y_rows=y_rows, h_bits=h_bits, mass_y=mass_y, slack_h=slack_h)


def combine(y_rows: np.ndarray, row_of: np.ndarray, w: np.ndarray, T: int, k: int):
    """y[t] = sum_j w[t, j] * O[row_of[t*k + j]] in fp64; out = bf16_rne(y)
    (one rounding, at the end). Returns (y float64 [T, d], out bits uint16)."""
    ro = np.asarray(row_of, dtype=np.int64).reshape(T, k)
    y = np.zeros((T, y_rows.shape[1]))
    for j in range(k):
        y += w[:, j:j + 1] * y_rows[ro[:, j]]
    return y, F.bf16_rne_bits(y)


@dataclass
class MoEResult:
    ids: np.ndarray
    w: np.ndarray
    rl: RowLists
    ffn: FFNResult
    y: np.ndarray          # float64 [T, d] before the final rounding
    out_bits: np.ndarray   # uint16 [T, d]
    mass: np.ndarray       # float64 [T, d]: sum_j w * mass_y
    slack: np.ndarray      # float64 [T, d]: sum_j w * slack_h


def moe_layer(inp) -> MoEResult:
    """The whole layer: route, row lists, expert FFN for every row, combine."""
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    ex = experts_dict(inp)
    validate_moe(T, d, f, E, k, inp.x, inp.logits, ex)
    ids, w = route(inp.logits, k)
    rl = row_lists(ids, E)
    ffn = expert_ffn(inp.x, T, d, f, E, k, ex, rl)
    y, out_bits = combine(ffn.y_rows, rl.row_of, w, T, k)
    ro = rl.row_of.astype(np.int64).reshape(T, k)
    mass = np.zeros((T, d))
    slack = np.zeros((T, d))
    for j in range(k):
        mass += w[:, j:j + 1] * ffn.mass_y[ro[:, j]]
        slack += w[:, j:j + 1] * ffn.slack_h[ro[:, j]]
    return MoEResult(ids, w, rl, ffn, y, out_bits, mass, slack)


def moe_tokens(inp, tokens, ids=None, w=None, rl=None, map_fn=map) -> MoEResult:
    """The layer's output for a subset of tokens only (each token's output needs
    only its own k rows), for sampled checks at sizes where the whole layer
    would take too long on the CPU. Routing is computed for every token (it is
    needed for the row lists)."""
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    ex = experts_dict(inp)
    if ids is None:
        validate_moe(T, d, f, E, k, inp.x, inp.logits, ex)
        ids, w = route(inp.logits, k)
        rl = row_lists(ids, E)
    tokens = np.asarray(tokens, dtype=np.int64)
    assign = (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    rows = rl.row_of[assign].astype(np.int64)
    ffn = expert_ffn(inp.x, T, d, f, E, k, ex, rl, rows=rows, map_fn=map_fn)
    nt = tokens.size
    yr = ffn.y_rows.reshape(nt, k, d)
    ws = w[tokens]
    y = np.einsum("tj,tjd->td", ws, yr)
    mass = np.einsum("tj,tjd->td", ws, ffn.mass_y.reshape(nt, k, d))
    slack = np.einsum("tj,tjd->td", ws, ffn.slack_h.reshape(nt, k, d))
    return MoEResult(ids, w, rl, ffn, y, F.bf16_rne_bits(y), mass, slack)


def silu_scalar(g: float) -> float:
    """Scalar silu for brute-force checks."""
    if g >= 0:
        return g / (1.0 + math.exp(-g))
    eg = math.exp(g)
    return g * eg / (1.0 + eg)
