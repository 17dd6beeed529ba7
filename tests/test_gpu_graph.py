"""Few-token calls captured in a HIP graph (torch.cuda.CUDAGraph, through the C ABI): every
replay gives the bits of a direct call on the inputs it sees, also when the activations
change between replays -- each replay takes a fresh tag for the words its workgroups hand
over (H, and the layer's expert rows) from the workspace, so no replay can take words an
earlier one left. Eager work and synchronizations run between the replays."""
import numpy as np
import pytest

import workloads

from gpu_util import say, upload_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


def _xs(inp, n=3):
    """The configuration's activations and n - 1 other draws of the same shape."""
    import torch
    out = [torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)]
    for s in range(1, n):
        o = workloads.make_moe(inp.T, inp.d, inp.f, inp.E, inp.k, seed=100 + s, config_id=97, experts=False)
        out.append(torch.from_numpy(o.x.view(np.int16)).cuda().view(torch.bfloat16))
    return out


def _replay_and_check(g, x_static, xs, got, refs, label):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    for rep, i in enumerate((1, 0, 2, 2, 1, 0)):
        x_static.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        assert M.async_status() == 0
        same = torch.equal(got.view(torch.int32) if got.dtype == torch.float32 else got.view(torch.int16),
                           refs[i].view(torch.int32) if got.dtype == torch.float32 else refs[i].view(torch.int16))
        say(f"{label}: replay {rep} on input {i}: {'same bits' if same else 'DIFFERENT'}")
        assert same
        # eager work between replays
        _ = (xs[i].float() * 2).sum().item()


def test_graph_expert_ffn_few_tokens():
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    x0, logits, ex = upload_moe(inp)
    xs = _xs(inp)
    ids, w, off, srows, rof = M.route_topk(logits, inp.k)
    refs = [M.expert_ffn_nvfp4(x, ex, off, srows, inp.k).clone() for x in xs]
    x_s = xs[0].clone()
    y_s = torch.empty((inp.T * inp.k, inp.d), dtype=torch.float32, device="cuda")
    ws = torch.zeros((M.expert_ffn_workspace(inp.T, inp.d, inp.f, inp.E, inp.k),), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (device caches, attributes)
        M.expert_ffn_nvfp4(x_s, ex, off, srows, inp.k, out=y_s, workspace=ws, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.expert_ffn_nvfp4(x_s, ex, off, srows, inp.k, out=y_s, workspace=ws, check=False)
    _replay_and_check(g, x_s, xs, y_s, refs, "expert_ffn_nvfp4 (decode)")


def test_graph_no_alloc_entry():
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    x0, logits, ex = upload_moe(inp)
    xs = _xs(inp)
    ids, w, off, srows, rof = M.route_topk(logits, inp.k)
    refs = [M.expert_ffn_nvfp4(x, ex, off, srows, inp.k).clone() for x in xs]
    x_s = xs[0].clone()
    y_s = torch.empty((inp.T * inp.k, inp.d), dtype=torch.float32, device="cuda")
    M.expert_ffn_nvfp4_scratch(x_s, ex, off, srows, inp.k, out=y_s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.expert_ffn_nvfp4_scratch(x_s, ex, off, srows, inp.k, out=y_s)
    _replay_and_check(g, x_s, xs, y_s, refs, "expert_ffn_nvfp4_scratch")


def test_graph_layer_one_launch():
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    sh = workloads.shared_config("decode")
    x0, logits, ex = upload_moe(inp)
    sex = M.NVFP4Experts.from_numpy(sh, "cuda")
    glog = torch.zeros((inp.T, 1), dtype=torch.float32, device="cuda")
    xs = _xs(inp)
    refs = [M.layer_nvfp4(logits, x, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x).clone() for x in xs]
    x_s = xs[0].clone()
    out = torch.empty((inp.T, inp.d), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros((M.layer_workspace(inp.T, inp.d, inp.f, inp.E, inp.k, True),), dtype=torch.uint8, device="cuda")
    M.layer_nvfp4(logits, x_s, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x_s, out=out, workspace=ws,
                  check=False)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.layer_nvfp4(logits, x_s, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x_s, out=out,
                      workspace=ws, check=False)
    _replay_and_check(g, x_s, xs, out, refs, "layer_nvfp4 (decode, shared expert, residual)")
