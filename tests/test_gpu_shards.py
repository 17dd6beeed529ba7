"""One GPU's share of the layer under the two ways it would shard (the exchanges between
GPUs are not part of this build; the share's kernels are, at their real shapes):

* expert parallelism (EP = 8, a prompt batch): a GPU owns E/8 consecutive experts and runs
  the FFN on the rows routed to them, gathered (k = 1 a row). Its rows must equal the same
  rows of the whole layer's call bit for bit -- the same experts, rows and tiles;
* tensor parallelism over f (TP = 8, decode): a GPU holds f/8 features of every expert and
  computes the partial layer an all-reduce would sum; checked against the CPU oracle."""
import numpy as np
import pytest

import workloads
from oracle import moe

from gpu_util import check_layer_full, run_moe, say, upload_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


def ep_share_call(x, ex, off, srows, k, ep, rank):
    """The FFN of rank `rank`'s experts on the rows routed to them: (y_local, p0, p1) with
    rows p0 .. p1 - 1 of the whole call's row list."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    E = ex.E
    e0, e1 = rank * E // ep, (rank + 1) * E // ep
    offs = off.cpu().numpy()
    p0, p1 = int(offs[e0]), int(offs[e1])
    toks = srows[p0:p1].long() // k
    x_loc = x.index_select(0, toks).contiguous()
    off_loc = (off[e0:e1 + 1] - p0).contiguous()
    rows_loc = torch.arange(p1 - p0, dtype=torch.int32, device=x.device)
    ex_loc = M.NVFP4Experts(*[getattr(ex, n)[e0:e1].contiguous() for n in
                              ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")])
    return M.expert_ffn_nvfp4(x_loc, ex_loc, off_loc, rows_loc, 1), p0, p1


@pytest.mark.parametrize("name", ["prompt", "long_prompt"])
def test_ep_share_rows_equal_the_whole_call(name):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.moe_config(name)
    x, logits, ex = upload_moe(inp)
    ids, w, off, srows, rof = M.route_topk(logits, inp.k)
    y_all = M.expert_ffn_nvfp4(x, ex, off, srows, inp.k)
    counts = np.diff(off.cpu().numpy())
    per_rank = [int(counts[r * inp.E // 8:(r + 1) * inp.E // 8].sum()) for r in range(8)]
    heavy = int(np.argmax(per_rank))
    say(f"{name} EP=8 rows a rank: {per_rank}")
    for rank in sorted({0, heavy}):
        y_loc, p0, p1 = ep_share_call(x, ex, off, srows, inp.k, 8, rank)
        torch.cuda.synchronize()
        same = torch.equal(y_loc.view(torch.int32), y_all[p0:p1].view(torch.int32))
        say(f"{name} EP=8 rank {rank}: {p1 - p0} rows, {'same bits' if same else 'DIFFERENT'} as the whole call")
        assert p1 - p0 > 16 and same


@pytest.mark.parametrize("rank", [0, 7])
def test_tp_share_decode_layer(rank):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.tp_share(workloads.moe_config("decode"), 8, rank)
    say(f"decode TP=8 rank {rank}: f={inp.f}")
    check_layer_full(inp, run_moe(inp), f"decode tp8 rank {rank}")
    # the one-launch layer on the share: the same bits as the separate entry points
    x, logits, ex = upload_moe(inp)
    ids, w, off, srows, rof = M.route_topk(logits, inp.k)
    ref = M.combine(M.expert_ffn_nvfp4(x, ex, off, srows, inp.k), rof, w)
    got = M.layer_nvfp4(logits, x, ex, inp.k)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
