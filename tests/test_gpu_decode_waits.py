"""The few-token launch's waits (through the C ABI): a down-product workgroup whose
expert's H slices are still missing after a number of polls computes those gate/up
items itself (same code, same bits), so the waits end whatever else runs on the GPU; a
wait that gives up (a guard) is reported by moe_async_status by name. Every kernel here
exits normally: both paths are forced from the host through moe_set_wait_limits, never
by a fault or a hang."""
import numpy as np
import pytest

import workloads
from oracle import band, moe

from gpu_util import check_band, check_layer_full, check_routing, run_moe, say, upload_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()
    assert M.async_status() == 0, "a wait expired before these tests"


def _fused(inp, x, logits, ex, ws=None):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    (ids, w, off, sr, ro), y = M.route_expert_ffn_nvfp4(logits, x, ex, inp.k, workspace=ws)
    out = M.combine(y, ro, w)
    return dict(ids=ids, w=w, offsets=off, sorted_rows=sr, row_of=ro, y_rows=y, out=out)


def _np(res):
    import torch
    r = {k: v.cpu().numpy() for k, v in res.items() if k != "out"}
    r["out"] = res["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    return r


def test_forced_give_up_is_reported():
    """Limits (0, 0): a down-product workgroup that finds an H slice missing gives up at
    once (no computing it itself), writes NaN in its tile and raises the flag;
    moe_async_status reports MOE_E_WAIT_EXPIRED exactly when some element is NaN, every
    element written is right, and the report clears the flag. With the limits restored
    the same call is whole."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config("decode")
    x, logits, ex = upload_moe(inp)
    ref = moe.moe_layer(inp)
    seen_expired = 0
    prev = M.set_wait_limits(0, 0)
    try:
        for i in range(5):
            res = _np(_fused(inp, x, logits, ex))
            st = M.async_status()
            nan = np.isnan(res["y_rows"])
            say(f"limits (0, 0), call {i}: status {st}, NaN elements {int(nan.sum())} of {nan.size}")
            assert st in (0, 7)
            assert (st == 7) == bool(nan.any())
            seen_expired += st == 7
            # a down item that gave up leaves NaN in its (expert rows x 128 columns); every
            # element written is right
            ok = ~nan
            check_band(band.classify_f32(res["y_rows"][ok], ref.ffn.y_rows[ok], ref.ffn.mass_y[ok], ref.ffn.slack_h[ok]),
                       f"decode, forced give-up, call {i}", f"y_rows ({int(ok.sum())} elements not given up)")
    finally:
        M.set_wait_limits(*prev)
    assert M.async_status() == 0
    say(f"calls with a wait given up: {seen_expired} of 5")
    assert seen_expired > 0, "no wait gave up: the forced exit path was not exercised"
    res = _np(_fused(inp, x, logits, ex))
    assert M.async_status() == 0
    check_layer_full(inp, res, "decode after the limits are restored")


@pytest.mark.parametrize("name", ["decode", "tiny", "edge"])
def test_forced_stealing_same_bits(name):
    """Limits (0, default): every down-product workgroup that finds an H slice missing at
    its first look computes the missing gate/up items itself. The outputs are the same
    bits as with the default limits (and within the band), and no wait gives up."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    if name == "edge":
        inp = workloads.make_moe(16, 512, 256, 16, 4, seed=5, config_id=64, zipf=True, scale_codes="finite",
                                 tensor_scales="edge")
    else:
        inp = workloads.moe_config(name)
    x, logits, ex = upload_moe(inp)
    base = _np(_fused(inp, x, logits, ex))
    prev = M.set_wait_limits(0, M.wait_limits()[1])
    try:
        outs = [_np(_fused(inp, x, logits, ex)) for _ in range(5)]
        y2 = M.expert_ffn_nvfp4(x, ex, torch.from_numpy(base["offsets"]).cuda(),
                                torch.from_numpy(base["sorted_rows"]).cuda(), inp.k)
        torch.cuda.synchronize()
    finally:
        M.set_wait_limits(*prev)
    assert M.async_status() == 0
    check_layer_full(inp, outs[0], f"{name}, forced stealing")
    for i, r in enumerate(outs):
        for key in ("ids", "offsets", "sorted_rows", "row_of", "out"):
            assert np.array_equal(r[key], base[key]), (i, key)
        assert np.array_equal(r["y_rows"].view(np.uint32), base["y_rows"].view(np.uint32)), i
    assert np.array_equal(y2.cpu().numpy().view(np.uint32), base["y_rows"].view(np.uint32))
    say(f"{name}: 6 calls with forced stealing, bit-identical to the default")


@pytest.mark.parametrize("name", ["decode", "tiny"])
def test_decode_beside_other_work(name):
    """Few-token launches while a large matrix product runs on a second stream (so the
    launch's workgroups may not all be resident together): the same bits as alone, call
    after call, and no wait expires."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config(name)
    x, logits, ex = upload_moe(inp)
    alone = _np(_fused(inp, x, logits, ex))
    check_layer_full(inp, alone, f"{name} alone")
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    outs = []
    ws = torch.empty((M.expert_ffn_workspace(inp.T, inp.d, inp.f, inp.E, inp.k),), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(side):
            for _ in range(4):
                c = a @ b
        for _ in range(10):
            outs.append(_fused(inp, x, logits, ex, ws))
        main.wait_stream(side)
    torch.cuda.synchronize()
    del c
    assert M.async_status() == 0
    for i, o in enumerate(outs):
        r = _np(o)
        for key in ("ids", "offsets", "sorted_rows", "row_of", "out"):
            assert np.array_equal(r[key], alone[key]), (i, key)
        assert np.array_equal(r["y_rows"].view(np.uint32), alone["y_rows"].view(np.uint32)), i
    say(f"{name}: {len(outs)} calls beside a matrix product on a second stream, all bit-identical")
