"""The allocation-free expert FFN (moe_expert_ffn_nvfp4_scratch: H in the library's static
device scratch) against the workspace entry point moe_expert_ffn_nvfp4, through the C ABI:
calls in a row on one device, each smaller than the one before (the prompt configuration,
a smaller prompt-path batch, the decode configuration), every output bit for bit equal to
the workspace entry point's on the same inputs."""
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


def _compare(inp, where):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    need = M.expert_ffn_workspace(T, d, f, E, k)
    assert 0 < need <= M.SCRATCH_BYTES, need
    x, logits, ex = upload_moe(inp)
    ids, w, off, sr, ro = M.route_topk(logits, k)
    ref = M.expert_ffn_nvfp4(x, ex, off, sr, k)
    out = torch.full((T * k, d), float("nan"), dtype=torch.float32, device="cuda")
    M.expert_ffn_nvfp4_scratch(x, ex, off, sr, k, out)
    torch.cuda.synchronize()
    a = ref.cpu().numpy()
    b = out.cpu().numpy()
    assert not np.isnan(b).any(), f"{where}: rows left unwritten"
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{where}: differs from the workspace entry point"
    say(f"[{where}] no-alloc entry point: {b.size} fp32 outputs equal to the workspace entry point's (H {need} bytes)")


def test_no_alloc_calls_in_a_row():
    _compare(workloads.moe_config("prompt"), "prompt T=512 d=3072 f=1536 E=128 k=8")
    _compare(workloads.make_moe(300, 512, 256, 8, 2, seed=12, config_id=67, zipf=True), "T=300 d=512 f=256 E=8 k=2")
    _compare(workloads.moe_config("decode"), "decode T=4 d=2048 f=768 E=128 k=8")
    _compare(workloads.moe_config("tiny"), "tiny T=4 d=256 f=128 E=8 k=2")
