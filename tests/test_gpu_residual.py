"""GPU parity of the block's output with its residual stream (moe_combine_residual, through
the C ABI) against the CPU oracle: out = bf16_rne(x + sum_j w O + g S), with and without
the shared expert; a zero residual gives the values of the plain combine."""
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


def _run(inp, sh=None, zero_residual=False):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    x, logits, ex = upload_moe(inp)
    ids, w, off, srows, rof = M.route_topk(logits, inp.k)
    y_rows = M.expert_ffn_nvfp4(x, ex, off, srows, inp.k)
    s_rows = glog = None
    if sh is not None:
        sex = M.NVFP4Experts.from_numpy(sh, "cuda")
        wsg = torch.from_numpy(sh.w_sg.view(np.int16).reshape(1, -1)).cuda().view(torch.bfloat16)
        s_rows = M.shared_expert_nvfp4(x, sex)
        glog = M.router_logits(x, wsg)
    resid = torch.zeros_like(x) if zero_residual else x
    out = M.combine(y_rows, rof, w, shared_rows=s_rows, shared_gate_logit=glog, residual=resid)
    plain = M.combine(y_rows, rof, w, shared_rows=s_rows, shared_gate_logit=glog)
    torch.cuda.synchronize()
    return (out.view(torch.int16).cpu().numpy().view(np.uint16), plain.view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("name", ["tiny", "decode"])
@pytest.mark.parametrize("with_shared", [False, True])
def test_residual_full(name, with_shared):
    inp = workloads.moe_config(name)
    sh = workloads.shared_config(name) if with_shared else None
    say(f"residual {name} shared={with_shared}")
    got, _ = _run(inp, sh)
    base = oshared.moe_layer_shared(inp, sh) if with_shared else moe.moe_layer(inp)
    ref = block.add_residual(base, inp.x)
    check_band(band.classify(got, ref.out_bits, ref.mass, ref.slack), f"residual {name} shared={with_shared}")


@pytest.mark.parametrize("T,d,f,E,k", [(1, 64, 32, 4, 2), (17, 160, 96, 6, 3), (300, 256, 128, 8, 2)])
def test_residual_small(T, d, f, E, k):
    inp = workloads.make_moe(T, d, f, E, k, seed=4, config_id=94, zipf=True)
    sh = workloads.make_shared(d, f, seed=4, config_id=94)
    say(f"residual small T={T} d={d} f={f} E={E} k={k}")
    got, _ = _run(inp, sh)
    ref = block.add_residual(oshared.moe_layer_shared(inp, sh), inp.x)
    check_band(band.classify(got, ref.out_bits, ref.mass, ref.slack), f"residual small T{T}d{d}f{f}E{E}k{k}")


def test_residual_prompt_sampled():
    inp = workloads.moe_config("prompt")
    sh = workloads.shared_config("prompt")
    toks = np.sort(np.random.default_rng(6).choice(inp.T, size=24, replace=False))
    say(f"residual prompt, {toks.size} sampled tokens")
    got, _ = _run(inp, sh)
    ref = block.add_residual(oshared.moe_tokens_shared(inp, sh, toks), inp.x, toks)
    check_band(band.classify(got[toks], ref.out_bits, ref.mass, ref.slack), "residual prompt",
               f"out ({toks.size} sampled tokens)")


@pytest.mark.parametrize("with_shared", [False, True])
def test_zero_residual_is_the_plain_combine(with_shared):
    """x = 0 as the residual: the same values as the combine without it (bits may differ
    only in the sign of zero)."""
    from oracle import formats as F
    inp = workloads.moe_config("decode")
    sh = workloads.shared_config("decode") if with_shared else None
    got, plain = _run(inp, sh, zero_residual=True)
    assert np.array_equal(F.bf16_bits_to_f64(got), F.bf16_bits_to_f64(plain))
