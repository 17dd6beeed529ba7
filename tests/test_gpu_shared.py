"""GPU parity of the layer with a shared expert (through the C ABI) against the CPU
oracle: the shared expert's rows by moe_expert_ffn_nvfp4 with one expert, its gate
logit by moe_router_logits with the gate vector as a one-row router, and the add
folded into moe_combine_shared; every bf16 output within the band."""
import numpy as np
import pytest

import workloads
from oracle import band, shared as oshared

from gpu_util import check_band, say, upload_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


def _upload_shared(sh):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    ex = M.NVFP4Experts.from_numpy(sh, "cuda")
    wsg = torch.from_numpy(sh.w_sg.view(np.int16).reshape(1, -1)).cuda().view(torch.bfloat16)
    return ex, wsg


def _run(inp, sh, gated=True, side_stream=False):
    """route + routed FFN on the current stream; shared expert and gate logit on the same
    stream or on a side stream joined by events; then the combine with the shared add."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    x, logits, ex = upload_moe(inp)
    sex, wsg = _upload_shared(sh)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream() if side_stream else main
    ready = torch.cuda.Event()
    ready.record(main)
    with torch.cuda.stream(side):
        side.wait_event(ready)
        s_rows = M.shared_expert_nvfp4(x, sex)
        glog = M.router_logits(x, wsg) if gated else None
        done = torch.cuda.Event()
        done.record(side)
    ids, w, off, srows, rof = M.route_topk(logits, inp.k)
    y_rows = M.expert_ffn_nvfp4(x, ex, off, srows, inp.k)
    main.wait_event(done)
    out = M.combine(y_rows, rof, w, shared_rows=s_rows, shared_gate_logit=glog)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["tiny", "decode"])
@pytest.mark.parametrize("gated", [True, False])
def test_shared_layer_full(name, gated):
    inp = workloads.moe_config(name)
    sh = workloads.shared_config(name)
    say(f"shared layer {name} gated={gated}")
    got = _run(inp, sh, gated)
    ref = oshared.moe_layer_shared(inp, sh, gated=gated)
    check_band(band.classify(got, ref.out_bits, ref.mass, ref.slack), f"shared {name} gated={gated}")


@pytest.mark.parametrize("name,ntok", [("prompt", 16), ("long_prompt", 3)])
def test_shared_layer_sampled(name, ntok):
    inp = workloads.moe_config(name)
    sh = workloads.shared_config(name)
    say(f"shared layer {name}, {ntok} sampled tokens")
    got = _run(inp, sh, True)
    toks = np.sort(np.random.default_rng(4).choice(inp.T, size=ntok, replace=False))
    ref = oshared.moe_tokens_shared(inp, sh, toks)
    check_band(band.classify(got[toks], ref.out_bits, ref.mass, ref.slack), f"shared {name}", f"out ({ntok} sampled tokens)")


@pytest.mark.parametrize("T,d,f,E,k", [(1, 64, 32, 4, 2), (17, 160, 96, 6, 3), (40, 256, 128, 8, 2)])
def test_shared_layer_small(T, d, f, E, k):
    inp = workloads.make_moe(T, d, f, E, k, seed=3, config_id=92, zipf=True)
    sh = workloads.make_shared(d, f, seed=3, config_id=92)
    say(f"shared small T={T} d={d} f={f} E={E} k={k}")
    got = _run(inp, sh, True)
    ref = oshared.moe_layer_shared(inp, sh)
    check_band(band.classify(got, ref.out_bits, ref.mass, ref.slack), f"shared small T{T}d{d}f{f}E{E}k{k}")


@pytest.mark.parametrize("name", ["prompt", "T40", "decode", "tiny"])
def test_shared_side_stream_same_bits(name):
    """The shared expert on a side stream (joined by events) gives the same bits as on
    the main stream, on the prompt path and on the few-token path (whose single launch
    then overlaps another few-token launch: its workgroups take work in ticket order, so
    it does not need all of them resident at once)."""
    if name == "T40":
        inp = workloads.make_moe(40, 256, 128, 8, 2, seed=3, config_id=93, zipf=True)
        sh = workloads.make_shared(256, 128, seed=3, config_id=93)
    else:
        inp = workloads.moe_config(name)
        sh = workloads.shared_config(name)
    a = _run(inp, sh, True, side_stream=False)
    b = _run(inp, sh, True, side_stream=True)
    assert np.array_equal(a, b)
