"""CPU oracle for the routed NVFP4 mixture-of-experts FFN and the MXFP8 projection.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, fp64 statement of
what the GPU path must compute. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it; the product path never calls it and
shares no code, table or helper with it.

Sources. The method is the one the pages "bloomery 0.3.9" (release notes),
"bloomery 0.3.13" (release notes) and "NVIDIA FP4-Local checkpoints on DGX
Spark (TP=1, TP=2): format, model and speed plan in rounds #565" describe:
routed NVFP4 expert stacks (a gate, an up and a down product, each expert with
its own tensor scale) held in their stored bytes, routing of a whole batch in
one run, SwiGLU between gate/up and down, and a router-weighted combine of the
expert rows. The pages never print bit layouts or a worked example; where they
are silent the plainest reading is taken and listed in each function's
docstring. The E2M1 / E4M3 / E8M0 bit fields follow the OCP Microscaling
Formats (MX) v1.0 specification.

Modules:
  formats  - E2M1 / E4M3 / E8M0 decoders from bit fields; bfloat16 round to
             nearest even directly from float64.
  moe      - routing (top-k + renormalized softmax), stable row lists, NVFP4
             dequantization, the expert FFN, the combine, slack terms.
  mxfp8    - the MXFP8 block-scaled projection.
  band     - the per-element acceptance rule (strict / explained / fail).
  router   - the router projection and the routing policies.
  shared   - the shared expert beside the routed ones and its gate.
  block    - the block's output with the residual stream.
  w8a8     - MXFP8 activations (OCP MX conversion) and the W8A8 MXFP8 projection.

Parity status: every function is pinned by the not-GPU tests (closed forms,
brute force, library conversions, exact invariants). The end-to-end values at
the large shapes rest on those pins plus the oracle's own consistency: the pages
print no numeric example for this path.
"""
from . import formats, moe, mxfp8, band, block, w8a8  # noqa: F401
