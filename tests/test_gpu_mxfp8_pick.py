"""The few-row MXFP8 kernels and their pick per card (through the C ABI): every candidate
kernel is within the band for every row count it serves; mxfp8_autotune records a valid
pick for every M up to 16 at the projection's shape, and the calls that follow (4 and 8
rows) are within the band with it."""
import numpy as np
import pytest

import workloads
from oracle import band, mxfp8 as omx

from gpu_util import check_band, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()
    yield
    M.mxfp8_force_kernel(-1)


def _run(inp, rows):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    x = torch.from_numpy(inp.x[:rows].view(np.int16)).cuda().view(torch.bfloat16)
    y = M.mxfp8_gemm(x, torch.from_numpy(inp.w).cuda(), torch.from_numpy(inp.s).cuda())
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("kernel", [0, 1, 2])
def test_every_candidate_in_band(kernel):
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.make_mxfp8(16, 300, 1056, seed=5, config_id=75)
    _, ref, mass = omx.mxfp8_gemm(inp.x, inp.w, inp.s)
    M.mxfp8_force_kernel(kernel)
    try:
        for rows in range(1, 17):
            if kernel == 0 and rows > 8:
                continue
            got = _run(inp, rows)
            check_band(band.classify(got, ref[:rows], mass[:rows]), f"mxfp8 kernel {kernel} M={rows} N=300 K=1056")
    finally:
        M.mxfp8_force_kernel(-1)


@pytest.mark.timeout(300)
def test_autotune_at_the_projection_shape():
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.mxfp8_config(16)
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    picks, us = M.mxfp8_autotune(x, torch.from_numpy(inp.w).cuda(), torch.from_numpy(inp.s).cuda(), reps=10)
    say("picks by M: " + ", ".join(f"{m + 1}:{M.MXFP8_KERNELS[p]}" for m, p in enumerate(picks)))
    for m, (p, t) in enumerate(zip(picks, us)):
        assert p in (0, 1, 2) and not (p == 0 and m + 1 > 8)
        timed = [v for v in t if v == v]
        assert t[p] == min(timed), (m + 1, t)
    for rows in (4, 8):
        got = _run(inp, rows)
        _, ref, mass = omx.mxfp8_gemm(inp.x[:rows], inp.w, inp.s)
        check_band(band.classify(got, ref, mass), f"mxfp8 M={rows} N=12288 K=4096 (picked {M.MXFP8_KERNELS[picks[rows - 1]]})")
