"""The MoE block's output with the residual stream, plain fp64 CPU statement (test
infrastructure only).

Only tests/, the package's smoke check and the benchmark's CPU-baseline leg use this
module; the GPU path never imports it.

The routed experts and the shared expert beside them [FP4-Local checkpoints on DGX
Spark, §4 Round 1, #686] produce the block's update of a token; the block adds it to the
token's residual stream, and the pages fold the adds that follow a producer into that
producer [same page, §4 remaining items: prefill kernels folded into their producers,
SwiGLU and shared-expert add; §4 Round 1, #701: the sum folded into the combine].
Readings taken where the pages are silent (listed in the design notes):

1. The residual is the block's input activations x (bfloat16 [T, d]), the same rows the
   router and the experts read.
2. out[t] = bf16_rne(x[t] + sum_j w_tj O[row_of[t k + j]] + g_t S[t]): the residual is
   added before the single rounding, in exact arithmetic here (fp64 sum of exact
   values), in fp32 on the GPU.
3. Acceptance: the residual's magnitude joins the L1 mass of the sum (fp32 additions of
   it err by at most 2^-24 of the running sum, far inside the 2^-20 mass share).
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import moe


def add_residual(res: moe.MoEResult, x_bits, tokens=None) -> moe.MoEResult:
    """`res` (the routed layer, with or without the shared expert; all tokens, or the
    sampled `tokens` of moe_tokens) with each token's residual row x[t] added before the
    single rounding."""
    x = F.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    if tokens is not None:
        x = x[np.asarray(tokens, dtype=np.int64)]
    y = res.y + x
    return moe.MoEResult(res.ids, res.w, res.rl, res.ffn, y, F.bf16_rne_bits(y), res.mass + np.abs(x), res.slack)
