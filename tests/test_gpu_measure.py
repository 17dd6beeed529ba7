"""The benchmark's read-ceiling helper (moe_read_ceiling, through the C ABI) reads exactly
the ranges it is given: the xor of the words it returns equals the xor of every 32-bit
word of the ranges, computed on the host; ranges of several sizes, a piece spanning
ranges, one range."""
import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


@pytest.mark.parametrize("sizes", [[16], [4096, 65536 + 48, 16, 300000 - 300000 % 16], [1 << 22] * 3])
def test_read_ceiling_reads_its_ranges(sizes):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    rng = np.random.default_rng(len(sizes))
    bufs = [torch.from_numpy(rng.integers(0, 256, size=n, dtype=np.uint8)).cuda() for n in sizes]
    table = torch.tensor([(b.data_ptr(), b.numel()) for b in bufs], dtype=torch.int64, device="cuda")
    sink = torch.zeros((4096,), dtype=torch.int32, device="cuda")
    M.read_ceiling(table, sum(sizes), sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.uint32(0)
    for b in bufs:
        want ^= np.bitwise_xor.reduce(b.cpu().numpy().view(np.uint32))
    say(f"read ceiling over {sizes}: xor {got:#x}, host {want:#x}")
    assert got == want
