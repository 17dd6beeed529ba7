"""Shared expert beside the routed experts, plain fp64 CPU statement (test
infrastructure only).

Only tests/, the package's smoke check and the benchmark's CPU-baseline leg use
this module; the GPU path never imports it.

The pages run a shared expert beside the routed experts [FP4-Local checkpoints on
DGX Spark, §4 Round 1, #686], read its gate as the checkpoint's BF16 words [same
page, §4 Round 1, #732], and fold the shared-expert add into its producer, the
combine [same page, §4 Round 1, #701; §4 remaining items, prefill kernels folded
into their producers]. Readings taken where the pages are silent (listed in the
design notes):

1. The shared expert is a dense SwiGLU FFN of the routed experts' form and format
   (NVFP4 gate, up and down with E4M3 block scales and fp32 tensor scales) that
   every token passes through: S[t] = ts_d * (bf16_rne(silu(G) * U) . W_d^T).
2. The shared gate is g_t = sigmoid(x_t . w_sg) with w_sg bfloat16 [d].
3. The layer output is out[t] = bf16_rne(sum_j w_tj * O[row_of[t*k + j]] + g_t * S[t]):
   the shared row stays unrounded until the combine's single rounding.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import moe


def shared_dict(sh) -> dict:
    return {nm: getattr(sh, nm) for nm in
            ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")}


def shared_rows(x_bits, T: int, d: int, f: int, sh, tokens=None) -> moe.FFNResult:
    """S for every token (or the given tokens): the FFN of an expert that every token
    routes to (one expert, one choice per token, row p = token p)."""
    rl = moe.row_lists(np.zeros((T, 1), dtype=np.int32), 1)
    return moe.expert_ffn(x_bits, T, d, f, 1, 1, shared_dict(sh), rl, rows=tokens)


def shared_gate(x_bits, w_sg_bits, tokens=None):
    """g_t = sigmoid(x_t . w_sg) in fp64, and the logit's mass sum_i |x_ti w_i|."""
    x = F.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    if tokens is not None:
        x = x[np.asarray(tokens)]
    w = F.bf16_bits_to_f64(np.asarray(w_sg_bits, dtype=np.uint16))
    z = x @ w
    g = np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.abs(z))), np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))
    return g, np.abs(x) @ np.abs(w)


def gate_error_bound(d: int, g, gmass):
    """Largest |g32 - g| of a float32 gate: the float32 logit is within (d + 8) 2^-24 of
    its mass (any summation order, as for the router logits), which moves the sigmoid by
    at most a quarter of that (sigmoid' <= 1/4), plus 8 float32 ulps of the sigmoid
    itself (exp, add, divide)."""
    return 0.25 * (d + 8) * 2.0 ** -24 * np.asarray(gmass) + 8 * 2.0 ** -24 * np.asarray(g)


def add_shared(res: moe.MoEResult, x_bits, T, d, f, sh, tokens=None, gated: bool = True) -> moe.MoEResult:
    """The routed result `res` (whole layer, or the sampled `tokens` of moe_tokens) with
    the gated shared row added before the single rounding. The acceptance terms grow by
    g * mass_S and g * slack_S, plus the effect of the float32 gate logit: its error
    (at most (d + 8) 2^-24 of its mass, through sigmoid' <= 1/4) and a few ulps of the
    float32 sigmoid, times |S|. Ungated (``gated=False``): g = 1."""
    S = shared_rows(x_bits, T, d, f, sh, tokens)
    g, gmass = shared_gate(x_bits, sh.w_sg, tokens)
    if not gated:
        g, gmass = np.ones_like(g), np.zeros_like(gmass)
    y = res.y + g[:, None] * S.y_rows
    dg = gate_error_bound(d, g, gmass) if gated else np.zeros_like(g)
    mass = res.mass + g[:, None] * S.mass_y
    slack = res.slack + g[:, None] * S.slack_h + dg[:, None] * np.abs(S.y_rows)
    return moe.MoEResult(res.ids, res.w, res.rl, res.ffn, y, F.bf16_rne_bits(y), mass, slack)


def moe_layer_shared(inp, sh, gated: bool = True) -> moe.MoEResult:
    """The whole layer with the shared expert."""
    return add_shared(moe.moe_layer(inp), inp.x, inp.T, inp.d, inp.f, sh, gated=gated)


def moe_tokens_shared(inp, sh, tokens, gated: bool = True) -> moe.MoEResult:
    """Sampled tokens of the layer with the shared expert."""
    tokens = np.asarray(tokens, dtype=np.int64)
    return add_shared(moe.moe_tokens(inp, tokens), inp.x, inp.T, inp.d, inp.f, sh, tokens, gated=gated)
