"""GPU parity of the one-launch layer (moe_layer_nvfp4, through the C ABI): routing, the
routed experts, an optional shared expert and the combine with an optional residual, all in
one launch. Checked bit for bit against the same layer built from the separate entry points
(moe_route_topk, moe_expert_ffn_nvfp4, the shared expert's call, moe_combine*), and against
the CPU oracle within the band."""
import numpy as np
import pytest

import workloads
from oracle import band, block, moe, shared as oshared

from gpu_util import check_band, say, upload_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(inp, sh):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    x, logits, ex = upload_moe(inp)
    sex = glog = None
    if sh is not None:
        sex = M.NVFP4Experts.from_numpy(sh, "cuda")
        wsg = torch.from_numpy(sh.w_sg.view(np.int16).reshape(1, -1)).cuda().view(torch.bfloat16)
        glog = M.router_logits(x, wsg)
    return x, logits, ex, sex, glog


def _separate(x, logits, ex, k, sex, glog, resid):
    """The layer from the separate entry points."""
    import nvfp4_block_scaled_topk_amd as M
    ids, w, off, srows, rof = M.route_topk(logits, k)
    y = M.expert_ffn_nvfp4(x, ex, off, srows, k)
    s_rows = M.shared_expert_nvfp4(x, sex) if sex is not None else None
    out = M.combine(y, rof, w, shared_rows=s_rows, shared_gate_logit=glog if sex is not None else None,
                    residual=resid)
    return out, (ids, w, off, srows, rof)


def _route_bufs(T, E, k):
    import torch
    return (torch.full((T, k), -1, dtype=torch.int32, device="cuda"),
            torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((E + 1,), -1, dtype=torch.int32, device="cuda"),
            torch.full((T * k,), -1, dtype=torch.int32, device="cuda"),
            torch.full((T * k,), -1, dtype=torch.int32, device="cuda"))


def _check_same(inp, sh, with_resid, label):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    x, logits, ex, sex, glog = _inputs(inp, sh)
    resid = x if with_resid else None
    ref, rref = _separate(x, logits, ex, inp.k, sex, glog, resid)
    rb = _route_bufs(inp.T, inp.E, inp.k)
    got = M.layer_nvfp4(logits, x, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=resid, route_out=rb)
    torch.cuda.synchronize()
    assert M.async_status() == 0
    for a_, b_, nm in zip(rb, rref, ("ids", "w", "offsets", "sorted_rows", "row_of")):
        assert torch.equal(a_, b_), f"{label}: routing output {nm} differs"
    gb, rbits = _bits(got), _bits(ref)
    ndiff = int((gb != rbits).sum())
    say(f"{label}: one launch vs separate entry points: {ndiff} of {gb.size} bf16 elements differ")
    assert ndiff == 0
    return gb


@pytest.mark.parametrize("name", ["tiny", "decode"])
@pytest.mark.parametrize("with_shared", [False, True])
@pytest.mark.parametrize("with_resid", [False, True])
def test_layer_configs(name, with_shared, with_resid):
    inp = workloads.moe_config(name)
    sh = workloads.shared_config(name) if with_shared else None
    label = f"layer {name} shared={with_shared} residual={with_resid}"
    got = _check_same(inp, sh, with_resid, label)
    base = oshared.moe_layer_shared(inp, sh) if with_shared else moe.moe_layer(inp)
    ref = block.add_residual(base, inp.x) if with_resid else base
    check_band(band.classify(got, ref.out_bits, ref.mass, ref.slack), label)


@pytest.mark.parametrize("T,d,f,E,k", [(1, 64, 32, 4, 2), (3, 160, 96, 6, 3), (16, 1024, 1024, 256, 16),
                                       (7, 4096, 1024, 64, 8), (5, 2048, 768, 8, 8), (16, 224, 64, 32, 1)])
def test_layer_shapes(T, d, f, E, k):
    """Ragged column tiles (d not a multiple of 128), one row an expert, every expert chosen
    (E = k), the size limits (T = 16, E = 256, k = 16; d = 4096), top-1."""
    inp = workloads.make_moe(T, d, f, E, k, seed=5, config_id=95, zipf=True)
    sh = workloads.make_shared(d, f, seed=5, config_id=95)
    label = f"layer T={T} d={d} f={f} E={E} k={k}"
    got = _check_same(inp, sh, True, label)
    ref = block.add_residual(oshared.moe_layer_shared(inp, sh), inp.x)
    check_band(band.classify(got, ref.out_bits, ref.mass, ref.slack), label)


def test_layer_stacked_router_logits():
    """The shared gate's logit in column E of the router's output (one router launch for
    both): routing reads columns 0..E-1 only, the gate comes from column E."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    sh = workloads.shared_config("decode")
    x, logits, ex, sex, glog = _inputs(inp, sh)
    stacked = torch.cat([logits, glog], dim=1).contiguous()  # [T, E + 1]
    ref, _ = _separate(x, logits, ex, inp.k, sex, glog, x)
    got = M.layer_nvfp4(stacked, x, ex, inp.k, shared=sex, shared_gate_logit=stacked[:, inp.E:inp.E + 1],
                        residual=x)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_layer_repeat_and_forced_stealing():
    """Calls in a row on one workspace give the same bits (the tags of one call never match
    another's), and so does a call in which every down item that finds its H missing
    computes it itself (wait limits (0, default))."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    sh = workloads.shared_config("decode")
    x, logits, ex, sex, glog = _inputs(inp, sh)
    ws = torch.zeros((M.layer_workspace(inp.T, inp.d, inp.f, inp.E, inp.k, True),), dtype=torch.uint8, device="cuda")
    first = M.layer_nvfp4(logits, x, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x, workspace=ws).clone()
    for _ in range(3):
        again = M.layer_nvfp4(logits, x, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
    old = M.wait_limits()
    try:
        M.set_wait_limits(0, old[1])
        stolen = M.layer_nvfp4(logits, x, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x, workspace=ws)
        torch.cuda.synchronize()
    finally:
        M.set_wait_limits(*old)
    assert M.async_status() == 0
    assert torch.equal(stolen.view(torch.int16), first.view(torch.int16))


def test_layer_beside_other_work():
    """The one-launch layer on a side stream while a large bf16 matmul runs on another:
    same bits as alone (no wait depends on all of the launch's blocks being resident)."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    sh = workloads.shared_config("decode")
    x, logits, ex, sex, glog = _inputs(inp, sh)
    alone = M.layer_nvfp4(logits, x, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x).clone()
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for _ in range(4):
        c = a @ a
        with torch.cuda.stream(side):
            outs.append(M.layer_nvfp4(logits, x, ex, inp.k, shared=sex, shared_gate_logit=glog, residual=x))
        del c
    torch.cuda.synchronize()
    assert M.async_status() == 0
    for o in outs:
        assert torch.equal(o.view(torch.int16), alone.view(torch.int16))


def test_layer_refusals():
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("tiny")
    x, logits, ex, sex, glog = _inputs(inp, None)
    big = workloads.make_moe(17, 64, 32, 4, 2, seed=1, config_id=96)
    xb, lb, eb = upload_moe(big)
    with pytest.raises(M.MoEError, match="MOE_E_SHAPE"):  # more than 16 tokens
        M.layer_nvfp4(lb, xb, eb, big.k)
    assert M.layer_workspace(17, 64, 32, 4, 2) == 0
    with pytest.raises(M.MoEError, match="MOE_E_WORKSPACE"):
        M.layer_nvfp4(logits, x, ex, inp.k, workspace=torch.empty((16,), dtype=torch.uint8, device="cuda"))


def test_layer_workspace_not_zero_filled_is_reported():
    """A workspace whose arrival counters were not zero-filled: the launch combines nothing
    it cannot vouch for, every kernel exits normally, and moe_async_status names it; after a
    zero fill the same workspace gives the right bits."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    x, logits, ex, sex, glog = _inputs(inp, None)
    ref, _ = _separate(x, logits, ex, inp.k, None, None, None)
    ws = torch.full((M.layer_workspace(inp.T, inp.d, inp.f, inp.E, inp.k),), 1, dtype=torch.uint8, device="cuda")
    M.layer_nvfp4(logits, x, ex, inp.k, workspace=ws)
    torch.cuda.synchronize()
    assert M.async_status() == 7  # MOE_E_WAIT_EXPIRED
    ws.zero_()
    got = M.layer_nvfp4(logits, x, ex, inp.k, workspace=ws)
    torch.cuda.synchronize()
    assert M.async_status() == 0
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "decode", "prompt_small"])
def test_moe_layer_convenience(name):
    """moe_layer (route, FFN, combine in one call): one launch where the shape allows, the
    three entry points otherwise; the same bits as those entry points either way."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = (workloads.moe_config(name) if name != "prompt_small"
           else workloads.make_moe(40, 256, 128, 16, 4, seed=6, config_id=94, zipf=True))
    x, logits, ex, _, _ = _inputs(inp, None)
    ref, _ = _separate(x, logits, ex, inp.k, None, None, None)
    got = M.moe_layer(x, logits, ex, inp.k)
    torch.cuda.synchronize()
    assert M.async_status() == 0
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
