"""Seeded synthetic inputs for the routed NVFP4 MoE layer and the MXFP8 projection.

This module only draws random numbers and lays them out as stored bytes. It holds
none of the method's arithmetic (no decoding, routing, products or rounding of
the method): the oracle and the GPU path both consume exactly these arrays.

Every tensor has its own generator, ``numpy.random.default_rng([seed, config_id,
tensor_id])``, so a draw never depends on the order in which tensors are made.

Distributions (the workloads of the routed NVFP4 expert stacks the pages run on
the card and in the prompt GEMM, [FP4-Local checkpoints on DGX Spark, §4 Round 1,
#517 and #545]; the pages' real prompts and trained weights are not available,
so these synthetic draws stand in for them):

* activations x: float32 N(0,1), converted to bfloat16 by torch's own
  float32 -> bfloat16 conversion (a library routine), returned as uint16 bits;
* router logits: float32 N(0,1), plus for the skewed configurations a Zipf
  bias ``-s * ln(r_e)`` with s = 1.1 and ranks ``r_e = 1 + pi(e)`` for a seeded
  permutation ``pi`` (a constant shift of all logits is dropped: it changes
  neither the selection nor the softmax);
* NVFP4 codes: uniform random bytes, so both nibbles are uniform over the 16
  E2M1 codes;
* NVFP4 block scales: uniform over the 49 E4M3 codes 0x18..0x48, whose values
  span [2^-4, 2^2];
* per-expert tensor scales: float32 uniform on [0.5, 2], one per expert and
  projection;
* router matrix W_r (bfloat16 [E, d]): float32 N(0, 1/d), converted to bfloat16 by
  torch, so the logits of N(0,1) activations are about N(0,1); the router inputs
  are the activations of the MoE configuration with the same name;
* shared expert: one NVFP4 expert (codes, block scales and tensor scales drawn as for
  the routed experts, from streams of its own), and a shared-gate vector bfloat16 [d]
  drawn as float32 N(0, 1/d);
* MXFP8 weights: uniform over the 254 finite E4M3 codes (0x7F and 0xFF
  excluded); E8M0 block scales uniform over codes 121..129 (2^-6 .. 2^2).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids inside one configuration's seed sequence
_T_X, _T_LOGITS, _T_PERM = 0, 1, 2
_T_GQ, _T_GS, _T_GTS = 3, 4, 5
_T_UQ, _T_US, _T_UTS = 6, 7, 8
_T_DQ, _T_DS, _T_DTS = 9, 10, 11
_T_MX_W, _T_MX_S = 22, 23
_T_ROUTER_W, _T_ROUTER_BIAS = 24, 25
_T_SH_GQ, _T_SH_GS, _T_SH_GTS, _T_SH_UQ, _T_SH_US, _T_SH_UTS, _T_SH_DQ, _T_SH_DS, _T_SH_DTS, _T_SH_GATE = range(40, 50)
_T_MX_X0 = 30  # + index of the M value

ZIPF_S = 1.1
ZIPF_ALPHA = 1.0

MOE_CONFIGS = {
    # name: (config_id, T, d, f, E, k, zipf)
    "tiny": (0, 4, 256, 128, 8, 2, False),
    "decode": (1, 4, 2048, 768, 128, 8, True),
    "prompt": (2, 512, 3072, 1536, 128, 8, True),
    "long_prompt": (3, 4096, 7168, 2048, 256, 8, True),
}
MXFP8_CONFIG = {"name": "mxfp8", "config_id": 4, "N": 12288, "K": 4096, "M": (1, 512)}


def _rng(seed: int, config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, config_id, tensor_id])


def _uniform_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def bf16_bits_from_normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draws, converted to bfloat16 by torch, as uint16 bits."""
    import torch

    f = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        f *= np.float32(std)
    b = torch.from_numpy(f).to(torch.bfloat16)
    return b.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class MoEInputs:
    """One MoE layer's inputs, every array as stored (see module docstring).

    Layouts (row-major):
      x        uint16 [T, d]       bfloat16 bits
      logits   float32 [T, E]
      gate_q   uint8 [E, f, d/2]   two E2M1 codes a byte, even element in the low nibble
      gate_s   uint8 [E, f, d/16]  E4M3 block scales, block = 16 consecutive K elements
      up_q / up_s                  as gate
      down_q   uint8 [E, d, f/2]
      down_s   uint8 [E, d, f/16]
      gate_ts / up_ts / down_ts    float32 [E] per-expert tensor scales
    """

    T: int
    d: int
    f: int
    E: int
    k: int
    x: np.ndarray
    logits: np.ndarray
    gate_q: np.ndarray
    gate_s: np.ndarray
    gate_ts: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    up_ts: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray
    down_ts: np.ndarray
    name: str = "custom"
    meta: dict = field(default_factory=dict)


def make_logits(T: int, E: int, seed: int, config_id: int, zipf: bool) -> np.ndarray:
    logits = _rng(seed, config_id, _T_LOGITS).standard_normal(size=(T, E), dtype=np.float32)
    if zipf:
        perm = _rng(seed, config_id, _T_PERM).permutation(E)
        ranks = 1.0 + perm.astype(np.float64)
        bias = (-ZIPF_ALPHA * ZIPF_S * np.log(ranks)).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
    return logits


# edge-case tensor scales: both signs, powers of two far from 1, and ordinary values
EDGE_TENSOR_SCALES = np.array([2.0 ** -8, -(2.0 ** -8), 2.0 ** 8, -(2.0 ** 8), -1.0, 0.75, -1.375, 3.0],
                              dtype=np.float32)


def _finite_e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform over the 254 finite E4M3 codes (0x7F and 0xFF, the NaN codes, excluded)."""
    j = rng.integers(0, 254, size=shape, dtype=np.int32)
    return np.where(j < 127, j, j + 1).astype(np.uint8)


def make_moe(T: int, d: int, f: int, E: int, k: int, seed: int = 0, config_id: int = 99,
             zipf: bool = False, name: str = "custom", experts: bool = True,
             scale_codes: str = "config", tensor_scales: str = "config") -> MoEInputs:
    """Draw one MoE layer's inputs. ``experts=False`` skips the weight draws
    (zero-size placeholders), for routing-only cases. Edge cases:
    ``scale_codes="finite"`` draws the E4M3 block scales uniformly over all 254 finite
    codes (zero, negative and subnormal scales, 448 included) instead of 0x18..0x48;
    ``tensor_scales="edge"`` draws each tensor scale from EDGE_TENSOR_SCALES."""
    if d % 32 or f % 32:
        raise ValueError("d and f must be multiples of 32")
    x = bf16_bits_from_normal(_rng(seed, config_id, _T_X), (T, d))
    logits = make_logits(T, E, seed, config_id, zipf)

    def codes(tid, shape):
        return _uniform_bytes(_rng(seed, config_id, tid), shape) if experts else np.zeros((0,), np.uint8)

    def scales(tid, shape):
        if not experts:
            return np.zeros((0,), np.uint8)
        if scale_codes == "finite":
            return _finite_e4m3_codes(_rng(seed, config_id, tid), shape)
        return _rng(seed, config_id, tid).integers(0x18, 0x49, size=shape, dtype=np.uint8)

    def tscale(tid):
        if tensor_scales == "edge":
            return _rng(seed, config_id, tid).choice(EDGE_TENSOR_SCALES, size=(E,)).astype(np.float32)
        return _rng(seed, config_id, tid).uniform(0.5, 2.0, size=(E,)).astype(np.float32)

    return MoEInputs(
        T=T, d=d, f=f, E=E, k=k, x=x, logits=logits,
        gate_q=codes(_T_GQ, (E, f, d // 2)), gate_s=scales(_T_GS, (E, f, d // 16)), gate_ts=tscale(_T_GTS),
        up_q=codes(_T_UQ, (E, f, d // 2)), up_s=scales(_T_US, (E, f, d // 16)), up_ts=tscale(_T_UTS),
        down_q=codes(_T_DQ, (E, d, f // 2)), down_s=scales(_T_DS, (E, d, f // 16)), down_ts=tscale(_T_DTS),
        name=name,
    )


def tp_share(inp: MoEInputs, tp: int, rank: int) -> MoEInputs:
    """One GPU's share of a layer under tensor parallelism over f: features
    rank * f/tp .. (rank + 1) * f/tp - 1 of every expert -- those rows of W_gate and W_up
    (with their block scales) and those columns of W_down (its K range: codes f/tp/2 and
    scales f/tp/16 of each row) -- and the same activations, logits and tensor scales.
    Array slicing only; f/tp must stay a multiple of 32."""
    fl = inp.f // tp
    if inp.f % tp or fl % 32:
        raise ValueError("f / tp must be a multiple of 32")
    a, b = rank * fl, (rank + 1) * fl
    return MoEInputs(
        T=inp.T, d=inp.d, f=fl, E=inp.E, k=inp.k, x=inp.x, logits=inp.logits,
        gate_q=np.ascontiguousarray(inp.gate_q[:, a:b]), gate_s=np.ascontiguousarray(inp.gate_s[:, a:b]),
        gate_ts=inp.gate_ts,
        up_q=np.ascontiguousarray(inp.up_q[:, a:b]), up_s=np.ascontiguousarray(inp.up_s[:, a:b]), up_ts=inp.up_ts,
        down_q=np.ascontiguousarray(inp.down_q[:, :, a // 2:b // 2]),
        down_s=np.ascontiguousarray(inp.down_s[:, :, a // 16:b // 16]), down_ts=inp.down_ts,
        name=f"{inp.name}_tp{tp}_rank{rank}")


def moe_config(name: str, seed: int = 0, experts: bool = True) -> MoEInputs:
    cid, T, d, f, E, k, zipf = MOE_CONFIGS[name]
    return make_moe(T, d, f, E, k, seed=seed, config_id=cid, zipf=zipf, name=name, experts=experts)


@dataclass
class MXFP8Inputs:
    """MXFP8 projection inputs, as stored.

      x  uint16 [M, K]      bfloat16 bits
      w  uint8 [N, K]       E4M3 codes (output-major, like a Linear weight)
      s  uint8 [N, K/32]    E8M0 block scales, block = 32 consecutive K elements
    """

    M: int
    N: int
    K: int
    x: np.ndarray
    w: np.ndarray
    s: np.ndarray
    name: str = "custom"


def make_mxfp8_weights(N: int, K: int, seed: int = 0, config_id: int = 99, e8m0=(121, 129)):
    """E4M3 weights uniform over the 254 finite codes; E8M0 scales uniform over the codes
    e8m0[0]..e8m0[1] (121..129: 2^-6 .. 2^2)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    w = _finite_e4m3_codes(_rng(seed, config_id, _T_MX_W), (N, K))
    s = _rng(seed, config_id, _T_MX_S).integers(e8m0[0], e8m0[1] + 1, size=(N, K // 32), dtype=np.uint8)
    return w, s


def make_mxfp8(M: int, N: int, K: int, seed: int = 0, config_id: int = 99, name: str = "custom",
               m_index: int = 0, e8m0=(121, 129)) -> MXFP8Inputs:
    w, s = make_mxfp8_weights(N, K, seed, config_id, e8m0)
    x = bf16_bits_from_normal(_rng(seed, config_id, _T_MX_X0 + m_index), (M, K))
    return MXFP8Inputs(M=M, N=N, K=K, x=x, w=w, s=s, name=name)


def mxfp8_config(M: int, seed: int = 0) -> MXFP8Inputs:
    """The MXFP8 projection's weights (N=12288, K=4096) with M activation rows: M = 1 and
    512 are the configuration's own; 2..16 (a few columns, for the per-card kernel pick)
    draw their activations from streams of their own."""
    c = MXFP8_CONFIG
    if M not in c["M"] and not 1 <= M <= 16:
        raise ValueError(f"M must be one of {c['M']} or in 1..16")
    m_index = c["M"].index(M) if M in c["M"] else 100 + M
    return make_mxfp8(M, c["N"], c["K"], seed=seed, config_id=c["config_id"], name=f"mxfp8_M{M}", m_index=m_index)


@dataclass
class RouterInputs:
    """The router projection's inputs: x uint16 [T, d] and w_r uint16 [E, d], bfloat16 bits."""
    name: str
    T: int
    d: int
    E: int
    x: np.ndarray
    w_r: np.ndarray


def make_router(T: int, d: int, E: int, seed: int = 0, config_id: int = 99, name: str = "custom") -> RouterInputs:
    x = bf16_bits_from_normal(_rng(seed, config_id, _T_X), (T, d))
    w_r = bf16_bits_from_normal(_rng(seed, config_id, _T_ROUTER_W), (E, d), std=float(1.0 / np.sqrt(d)))
    return RouterInputs(name, T, d, E, x, w_r)


def router_config(name: str, seed: int = 0) -> RouterInputs:
    """The router projection of a MoE configuration: the same activations (same seed
    stream as that configuration's x), and a router matrix of E rows of length d."""
    cid, T, d, f, E, k, zipf = MOE_CONFIGS[name]
    return make_router(T, d, E, seed=seed, config_id=cid, name=name)


def make_route_bias(E: int, seed: int = 0, config_id: int = 99, scale: float = 1.0, ties: bool = False) -> np.ndarray:
    """A correction bias, float32 [E]: scale * N(0,1), or with ``ties`` rounded to
    multiples of 1/2 (so biased keys tie often)."""
    b = _rng(seed, config_id, _T_ROUTER_BIAS).standard_normal(size=E, dtype=np.float32)
    if ties:
        b = np.round(b * 2) / 2
    return (b * np.float32(scale)).astype(np.float32)


@dataclass
class SharedInputs:
    """A shared expert beside the routed ones: one NVFP4 expert (arrays with a leading
    expert axis of 1, layouts as in MoEInputs) and the shared-gate vector w_sg uint16 [d]
    (bfloat16 bits)."""
    d: int
    f: int
    gate_q: np.ndarray
    gate_s: np.ndarray
    gate_ts: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    up_ts: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray
    down_ts: np.ndarray
    w_sg: np.ndarray


def make_shared(d: int, f: int, seed: int = 0, config_id: int = 99) -> SharedInputs:
    def codes(tid, shape):
        return _uniform_bytes(_rng(seed, config_id, tid), shape)

    def scales(tid, shape):
        return _rng(seed, config_id, tid).integers(0x18, 0x49, size=shape, dtype=np.uint8)

    def tscale(tid):
        return _rng(seed, config_id, tid).uniform(0.5, 2.0, size=(1,)).astype(np.float32)

    return SharedInputs(
        d=d, f=f,
        gate_q=codes(_T_SH_GQ, (1, f, d // 2)), gate_s=scales(_T_SH_GS, (1, f, d // 16)), gate_ts=tscale(_T_SH_GTS),
        up_q=codes(_T_SH_UQ, (1, f, d // 2)), up_s=scales(_T_SH_US, (1, f, d // 16)), up_ts=tscale(_T_SH_UTS),
        down_q=codes(_T_SH_DQ, (1, d, f // 2)), down_s=scales(_T_SH_DS, (1, d, f // 16)), down_ts=tscale(_T_SH_DTS),
        w_sg=bf16_bits_from_normal(_rng(seed, config_id, _T_SH_GATE), (d,), std=float(1.0 / np.sqrt(d))),
    )


def shared_config(name: str, seed: int = 0) -> SharedInputs:
    """The shared expert of a MoE configuration (same d and f)."""
    cid, T, d, f, E, k, zipf = MOE_CONFIGS[name]
    return make_shared(d, f, seed=seed, config_id=cid)

