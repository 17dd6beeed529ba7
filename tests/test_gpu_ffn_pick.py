"""The few-token path of moe_expert_ffn_nvfp4 picked per card (moe_ffn_autotune, through the
C ABI): both paths -- the one-launch decode kernel and the two weight-streaming kernels --
match the CPU oracle within the band at every row and output, the pick is one of the timed
paths, and later calls of that shape take it (the same bits as the path forced)."""
import numpy as np
import pytest

import workloads

from gpu_util import check_layer_full, run_moe, say, upload_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()
    yield
    M.ffn_force_path(-1)


# decode config; one expert every token routes to (the shared expert's call); the size
# limits of the decode kernel; a width past them (streaming path only); one token
SHAPES = [("decode", None), ("shared", (4, 2048, 768, 1, 1)), ("limits", (16, 1024, 1024, 64, 8)),
          ("wide", (4, 7168, 2048, 32, 8)), ("one", (1, 256, 128, 8, 2))]


def _inp(name, shape):
    if shape is None:
        return workloads.moe_config(name)
    T, d, f, E, k = shape
    return workloads.make_moe(T, d, f, E, k, seed=8, config_id=98, zipf=E > 8)


@pytest.mark.parametrize("name,shape", SHAPES)
@pytest.mark.parametrize("path", [0, 1])
def test_each_path_matches_the_oracle(name, shape, path):
    import nvfp4_block_scaled_topk_amd as M
    inp = _inp(name, shape)
    say(f"ffn path {M.FFN_PATHS[path]}: {name} T={inp.T} d={inp.d} f={inp.f} E={inp.E} k={inp.k}")
    M.ffn_force_path(path)
    try:
        res = run_moe(inp)
    finally:
        M.ffn_force_path(-1)
    check_layer_full(inp, res, f"ffn path {path} {name}")


@pytest.mark.parametrize("name,shape", SHAPES)
def test_autotune_records_a_timed_path(name, shape):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = _inp(name, shape)
    x, logits, ex = upload_moe(inp)
    ids, w, off, srows, rof = M.route_topk(logits, inp.k)
    pick, us = M.ffn_autotune(x, ex, off, srows, inp.k, reps=10)
    say(f"ffn pick {name}: {M.FFN_PATHS[pick]}; us {us}")
    assert pick in (0, 1)
    assert us[1] > 0 and (us[0] > 0 or np.isnan(us[0]))
    if name == "wide":  # past the decode kernel's size limits: only the streaming kernels
        assert pick == 1 and np.isnan(us[0])
    assert us[pick] <= min(v for v in us if not np.isnan(v))
    picked = M.expert_ffn_nvfp4(x, ex, off, srows, inp.k).clone()
    M.ffn_force_path(pick)
    try:
        forced = M.expert_ffn_nvfp4(x, ex, off, srows, inp.k)
    finally:
        M.ffn_force_path(-1)
    torch.cuda.synchronize()
    assert torch.equal(picked.view(torch.int32), forced.view(torch.int32))
