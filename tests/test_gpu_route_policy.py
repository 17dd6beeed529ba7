"""GPU parity of the routing policies and the correction bias (moe_route_topk_policy,
through the C ABI) against the CPU oracle: chosen ids and row lists bit for bit,
weights within (8 + n) * 2^-24 * |w| + 2^-40, with n the number of terms of the
normalizing sum (E for the softmax over all experts, k otherwise)."""
import numpy as np
import pytest

import workloads
from oracle import moe, router as orouter

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


def _check(logits, k, policy, bias, where):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    T, E = logits.shape
    bt = torch.from_numpy(bias).cuda() if bias is not None else None
    ids, w, off, sr, ro = M.route_topk(torch.from_numpy(logits).cuda(), k, policy=policy, bias=bt)
    torch.cuda.synchronize()
    ref_ids, ref_w = orouter.route_policy(logits, k, policy, bias)
    rl = moe.row_lists(ref_ids, E)
    assert np.array_equal(ids.cpu().numpy(), ref_ids), f"{where}: ids differ"
    assert np.array_equal(off.cpu().numpy(), rl.offsets), f"{where}: offsets differ"
    assert np.array_equal(sr.cpu().numpy(), rl.sorted_rows), f"{where}: sorted_rows differ"
    assert np.array_equal(ro.cpu().numpy(), rl.row_of), f"{where}: row_of differ"
    n = E if policy == orouter.SOFTMAX else k
    tol = (8 + n) * 2.0 ** -24 * np.abs(ref_w) + 2.0 ** -40
    err = np.abs(w.cpu().numpy().astype(np.float64) - ref_w)
    say(f"[{where}] max weight err {err.max():.3g}, worst err/bound {(err / tol).max():.3g}")
    assert np.all(err <= tol), f"{where}: weights beyond the bound"




# the layer shapes (row path: E <= 256, k <= 16), the wave path (E > 256 or k > 16),
# several token blocks, ragged E
SHAPES = [("decode", None), ("prompt", None), ("long_prompt", None),
          ("T130E1024k32", (130, 1024, 32)), ("T65E300k8", (65, 300, 8)), ("T3E7k3", (3, 7, 3))]


@pytest.mark.parametrize("policy", [0, 1, 2, 3])
@pytest.mark.parametrize("bias_kind", ["none", "bias", "bias_ties"])
@pytest.mark.parametrize("name,shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_route_policy(name, shape, policy, bias_kind):
    if shape is None:
        inp = workloads.moe_config(name, experts=False)
        logits, k = inp.logits, inp.k
    else:
        T, E, k = shape
        logits = workloads.make_logits(T, E, seed=7, config_id=90, zipf=True)
    E = logits.shape[1]
    if bias_kind == "bias_ties":
        logits = (np.round(logits * 2) / 2).astype(np.float32)  # ties between biased keys
    bias = None if bias_kind == "none" else workloads.make_route_bias(E, seed=11, config_id=90,
                                                                       ties=bias_kind == "bias_ties")
    _check(logits, k, policy, bias, f"{name} policy {policy} {bias_kind}")


def test_route_policy_wide_logits():
    """Logits spread over +-60 (sigmoid and softmax tails underflow in float32)."""
    logits = (workloads.make_logits(40, 64, seed=8, config_id=91, zipf=False) * 20).astype(np.float32)
    for policy in (0, 1, 2, 3):
        _check(logits, 6, policy, workloads.make_route_bias(64, seed=12, config_id=91, scale=10.0), f"wide policy {policy}")
