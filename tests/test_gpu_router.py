"""GPU parity of the router projection (through the C ABI) against the CPU oracle.

Every logit must lie within the fp32 summation bound (d + 8) * 2^-24 * mass of the
exact value; routing on the GPU's logits must then match the oracle's routing of
the same logits bit for bit."""
import numpy as np
import pytest

import workloads
from oracle import router as orouter

from gpu_util import check_routing, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


def _run(inp):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(inp.w_r.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full((inp.T, inp.E), float("nan"), dtype=torch.float32, device="cuda")
    M.router_logits(x, w, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(inp, got, where):
    exact, mass = orouter.router_logits(inp.x, inp.w_r)
    tol = orouter.router_tolerance(inp.d, mass)
    err = np.abs(got.astype(np.float64) - exact)
    worst = float(np.max(err / np.maximum(tol, 1e-300)))
    say(f"[router {where}] max |err| {err.max():.3g}, worst err/bound {worst:.3g}")
    assert not np.any(np.isnan(got)), f"{where}: unwritten logits"
    assert np.all(err <= tol), f"{where}: worst err/bound {worst:.3g}"


@pytest.mark.parametrize("name", ["tiny", "decode", "prompt", "long_prompt"])
def test_router_configs(name):
    inp = workloads.router_config(name)
    say(f"router {name}: T={inp.T} d={inp.d} E={inp.E}")
    _check(inp, _run(inp), name)


# one row, E not a multiple of 4, K shorter than the 8-way split, ragged tiles, many experts
ROUTER_SHAPES = [(1, 32, 1), (3, 96, 5), (33, 96, 33), (17, 64, 70), (100, 224, 7), (31, 32, 1000),
                 (65, 2048, 128), (200, 7168, 256)]


@pytest.mark.parametrize("T,d,E", ROUTER_SHAPES)
def test_router_shapes(T, d, E):
    inp = workloads.make_router(T, d, E, seed=5, config_id=80)
    say(f"router T={T} d={d} E={E}")
    _check(inp, _run(inp), f"T{T}d{d}E{E}")


def test_router_deterministic_and_routes():
    """Same inputs give the same bits twice; the GPU routing of the GPU logits equals
    the oracle's routing of those logits, bit for bit."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    for name, k in (("decode", 8), ("long_prompt", 8)):
        inp = workloads.router_config(name)
        a = _run(inp)
        b = _run(inp)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        ids, w, off, sr, ro = M.route_topk(torch.from_numpy(a).cuda(), k)
        torch.cuda.synchronize()
        res = dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), offsets=off.cpu().numpy(),
                   sorted_rows=sr.cpu().numpy(), row_of=ro.cpu().numpy())

        class _R:
            pass
        r = _R()
        r.logits, r.k, r.E = a, k, inp.E
        check_routing(r, res, f"router+route {name}")
