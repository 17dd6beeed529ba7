"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Routing indices, offsets and row lists must match bit for bit; every bf16 output
element must be within |gpu - oracle| <= 2e-3 + 2e-2 |oracle| (strict) or within
the documented slack (explained), never beyond (fail)."""
import numpy as np
import pytest

import workloads
from oracle import band, formats as F, moe, mxfp8 as omx

from gpu_util import (check_band, check_layer_full, check_layer_sampled, check_routing, cover_tokens, run_moe, say,
                      upload_moe)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_topk_amd as M
    M.lib()


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("name", ["tiny", "decode", "prompt", "long_prompt"])
def test_route_configs(name):
    inp = workloads.moe_config(name, experts=False)
    say(f"route {name}: T={inp.T} E={inp.E} k={inp.k}")
    import torch
    import nvfp4_block_scaled_topk_amd as M
    logits = torch.from_numpy(inp.logits).cuda()
    ids, w, off, sr, ro = M.route_topk(logits, inp.k)
    torch.cuda.synchronize()
    res = dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), offsets=off.cpu().numpy(),
               sorted_rows=sr.cpu().numpy(), row_of=ro.cpu().numpy())
    check_routing(inp, res, name)


# 1024 and 1025 tokens: 64 and 65 blocks of 16, the two sides of the switch from the one-level
# scan to the two-level one; 32768 tokens: 2048 blocks, more than one 1024-block chunk of
# the per-expert scan
ROUTE_EDGE = [(1, 1, 1), (1, 8, 8), (3, 64, 32), (16, 8, 2), (17, 8, 2), (33, 128, 8), (64, 7, 3), (65, 7, 3),
              (130, 1024, 32), (200, 65, 1), (129, 128, 8), (1000, 256, 8), (37, 33, 32), (1024, 256, 8),
              (1025, 256, 8), (32768, 256, 8), (20000, 1024, 32)]


@pytest.mark.parametrize("T,E,k", ROUTE_EDGE)
@pytest.mark.parametrize("ties", [False, True])
def test_route_edges(T, E, k, ties):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.make_moe(T, 32, 32, E, k, seed=3, config_id=50, zipf=not ties, experts=False)
    if ties:
        lg = np.round(inp.logits * 2).astype(np.float32)
        lg[lg == 0] = np.where(np.arange((lg == 0).sum()) % 2 == 0, -0.0, 0.0)
        inp.logits = lg
    say(f"route edge T={T} E={E} k={k} ties={ties}")
    ids, w, off, sr, ro = M.route_topk(torch.from_numpy(inp.logits).cuda(), k)
    torch.cuda.synchronize()
    res = dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), offsets=off.cpu().numpy(),
               sorted_rows=sr.cpu().numpy(), row_of=ro.cpu().numpy())
    check_routing(inp, res, f"T{T}E{E}k{k}")


# ---------------------------------------------------------------- whole layer
def test_layer_tiny():
    inp = workloads.moe_config("tiny")
    say("layer tiny")
    check_layer_full(inp, run_moe(inp), "tiny")


def test_layer_decode():
    inp = workloads.moe_config("decode")
    say("layer decode (T=4, d=2048, f=768, E=128, k=8)")
    check_layer_full(inp, run_moe(inp), "decode")


SMALL = [
    (1, 32, 32, 1, 1),       # single row; K tails only
    (3, 96, 64, 5, 2),       # decode path, K tail 96
    (16, 160, 96, 6, 3),     # decode path at its 16-row limit, ragged K
    (17, 160, 96, 6, 3),     # prompt path just above it
    (100, 224, 160, 12, 4),  # prompt path, ragged K and features
    (300, 256, 128, 4, 2),   # prompt path, experts with > 128 rows
    (40, 64, 32, 64, 8),     # many experts, few rows each
    (8, 2048, 768, 128, 8),  # decode shape with 8 tokens
    (200, 128, 64, 32, 4),   # prompt path: experts on both sides of the 16-row split
    (300, 512, 256, 6, 2),   # prompt path, d and f multiples of 256, ragged tiles
    (70, 256, 512, 3, 2),    # the same with f > d
    (150, 352, 320, 8, 2),   # prompt path, K stage counts 6 (half last stage) and 5
    (40, 2336, 2208, 8, 2),  # streaming kernels' line loads: chunk ranges of odd bounds, K tails
    (40, 2304, 2560, 8, 2),  # the same with K multiples of 256 (18 and 20 chunks): whole-line path
                             # with two-pair scale loads, waves' ranges starting on odd chunks
]


@pytest.mark.parametrize("T,d,f,E,k", SMALL)
def test_layer_small(T, d, f, E, k):
    inp = workloads.make_moe(T, d, f, E, k, seed=1, config_id=60, zipf=True)
    say(f"layer small T={T} d={d} f={f} E={E} k={k}")
    check_layer_full(inp, run_moe(inp), f"T{T}d{d}f{f}E{E}k{k}")


def test_layer_streaming_packing():
    """Experts of 4, 5..8 and 9..12 rows (uniform routing) on the whole-line streaming path
    (K multiples of 256, 18 and 20 chunks, waves' ranges starting on odd chunks): activation
    rows packed 4, 2 and 1 to a lane row; full outputs against the oracle."""
    inp = workloads.make_moe(40, 2304, 2560, 12, 2, seed=1, config_id=62, zipf=False)
    say("layer streaming packing T=40 d=2304 f=2560 E=12 k=2 (uniform routing)")
    check_layer_full(inp, run_moe(inp), "streaming packing T40d2304f2560E12k2")


def _covering_sample(inp, extra, seed):
    """Tokens covering every (expert, 128-row tile) of the grouped GEMM and every
    weight-streaming expert (first and last row of each), plus `extra` random tokens."""
    ids, _ = moe.route(inp.logits, inp.k)
    rl = moe.row_lists(ids, inp.E)
    toks = cover_tokens(rl.offsets, rl.sorted_rows, inp.k)
    more = np.random.default_rng(seed).choice(inp.T, size=extra, replace=False)
    return np.unique(np.concatenate([toks, more]))


@pytest.mark.timeout(900)
def test_layer_prompt_sampled():
    inp = workloads.moe_config("prompt")
    toks = _covering_sample(inp, 16, 0)
    say(f"layer prompt (T=512, d=3072, f=1536, E=128, k=8), {toks.size} tokens covering every tile")
    res = run_moe(inp)
    check_layer_sampled(inp, res, toks, "prompt")


@pytest.mark.timeout(900)
def test_layer_long_prompt_sampled():
    inp = workloads.moe_config("long_prompt")
    toks = _covering_sample(inp, 8, 1)
    say(f"layer long_prompt (T=4096, d=7168, f=2048, E=256, k=8), {toks.size} tokens covering every tile")
    res = run_moe(inp)
    check_layer_sampled(inp, res, toks, "long_prompt")


# E4M3 block scales over all 254 finite codes (zero, negative, subnormal, 448) and tensor
# scales of both signs including 2^-8 and 2^8: the decode path (T <= 16), the routing
# inside the FFN launch, the weight-streaming and grouped-GEMM prompt paths
EDGE = [(4, 256, 128, 8, 2), (16, 512, 256, 16, 4), (60, 256, 128, 8, 2), (300, 512, 256, 4, 2)]


@pytest.mark.parametrize("T,d,f,E,k", EDGE)
def test_layer_edge_codes(T, d, f, E, k):
    inp = workloads.make_moe(T, d, f, E, k, seed=5, config_id=64, zipf=True, scale_codes="finite",
                             tensor_scales="edge")
    say(f"layer edge codes T={T} d={d} f={f} E={E} k={k}")
    check_layer_full(inp, run_moe(inp), f"edge T{T}d{d}f{f}E{E}k{k}")
    if T <= 16:
        import torch
        import nvfp4_block_scaled_topk_amd as M
        x, logits, ex = upload_moe(inp)
        (ids, w, off, sr, ro), y = M.route_expert_ffn_nvfp4(logits, x, ex, k)
        out = M.combine(y, ro, w)
        torch.cuda.synchronize()
        res = dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), offsets=off.cpu().numpy(),
                   sorted_rows=sr.cpu().numpy(), row_of=ro.cpu().numpy(), y_rows=y.cpu().numpy(),
                   out=out.view(torch.int16).cpu().numpy().view(np.uint16))
        check_layer_full(inp, res, f"edge fused T{T}d{d}f{f}E{E}k{k}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T,d,f,E,k", [(4, 7168, 2048, 16, 8), (2, 4096, 2048, 8, 4)])
def test_layer_few_tokens_wide(T, d, f, E, k):
    """A few tokens with d > 4096 or f > 1024: past the one-launch few-token path, every
    expert takes the weight-streaming kernels (and the grouped GEMM has no tile)."""
    inp = workloads.make_moe(T, d, f, E, k, seed=6, config_id=65, zipf=True)
    say(f"layer few tokens, wide T={T} d={d} f={f} E={E} k={k}")
    check_layer_full(inp, run_moe(inp), f"wide T{T}d{d}f{f}E{E}k{k}")


def test_layer_deterministic_and_permutation():
    """Same inputs give the same bits twice; permuting the tokens permutes the
    outputs bit for bit (a row's result does not depend on its neighbours)."""
    for (T, d, f, E, k) in [(4, 256, 128, 8, 2), (60, 256, 128, 8, 2)]:
        inp = workloads.make_moe(T, d, f, E, k, seed=9, config_id=61, zipf=True)
        a = run_moe(inp)
        b = run_moe(inp)
        assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["y_rows"], b["y_rows"])
        perm = np.random.default_rng(2).permutation(T)
        inp2 = workloads.make_moe(T, d, f, E, k, seed=9, config_id=61, zipf=True)
        inp2.x = inp2.x[perm].copy()
        inp2.logits = inp2.logits[perm].copy()
        c = run_moe(inp2)
        assert np.array_equal(c["out"], a["out"][perm])
        assert np.array_equal(c["ids"], a["ids"][perm])


def test_decode_workspace_reuse():
    """The few-token path hands H over through tagged words in the workspace: one
    workspace, first filled with random bytes, then shared by consecutive calls with
    different routings and shapes (a larger call in between), each checked against the
    oracle -- words left by an earlier call must never be taken for this call's."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    from oracle import band, moe as omoe

    shapes = [(4, 256, 128, 8, 2), (3, 96, 64, 5, 2), (16, 160, 96, 6, 3), (40, 128, 64, 16, 4),
              (8, 512, 256, 16, 4), (4, 256, 128, 8, 2), (4, 256, 128, 8, 2), (16, 160, 96, 6, 3)]
    need = max(M.expert_ffn_workspace(T, d, f, E, k) for (T, d, f, E, k) in shapes)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    for i, (T, d, f, E, k) in enumerate(shapes):
        inp = workloads.make_moe(T, d, f, E, k, seed=20 + i, config_id=62, zipf=True)
        fused = T <= 16 and i % 2 == 1  # alternate the launch that routes its own tokens
        say(f"workspace reuse call {i}: T={T} d={d} f={f} E={E} k={k} fused={fused}")
        x, logits, ex = upload_moe(inp)
        y = torch.full((T * k, d), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            (ids, w, off, srows, rof), _ = M.route_expert_ffn_nvfp4(logits, x, ex, k, out=y, workspace=ws)
        else:
            ids, w, off, srows, rof = M.route_topk(logits, k)
            M.expert_ffn_nvfp4(x, ex, off, srows, k, out=y, workspace=ws)
        out = M.combine(y, rof, w)
        torch.cuda.synchronize()
        ref = omoe.moe_layer(inp)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        check_band(band.classify(got, ref.out_bits, ref.mass, ref.slack), f"workspace reuse call {i}")


# ---------------------------------------------------------------- MXFP8
def _run_mxfp8(inp):
    import torch
    import nvfp4_block_scaled_topk_amd as M
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(inp.w).cuda()
    s = torch.from_numpy(inp.s).cuda()
    y = M.mxfp8_gemm(x, w, s)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


# vector-ALU gemv (M <= 4), MFMA gemv (M <= 16) and tiled GEMM shapes: ragged M and N
# tiles, K tails of 32 (and of a 1 KB step), one stage, several tiles in each direction
MX_SMALL = [(1, 16, 32), (1, 100, 96), (3, 128, 4096), (16, 48, 160), (17, 130, 96), (200, 256, 288),
            (5, 33, 64), (129, 257, 64), (300, 600, 4128), (2, 70, 1056), (4, 9, 4096), (3, 1000, 32),
            # GEMM with the tile's scale rows preloaded (K a multiple of 512, <= 4096): ragged tiles
            (130, 200, 1024), (64, 193, 512), (300, 450, 2048)]


@pytest.mark.parametrize("M_,N,K", MX_SMALL)
def test_mxfp8_small(M_, N, K):
    inp = workloads.make_mxfp8(M_, N, K, seed=2, config_id=70)
    say(f"mxfp8 M={M_} N={N} K={K}")
    got = _run_mxfp8(inp)
    _, ref, mass = omx.mxfp8_gemm(inp.x, inp.w, inp.s)
    check_band(band.classify(got, ref, mass), f"mxfp8 {M_}x{N}x{K}")


@pytest.mark.parametrize("M_,N,K", [(1, 200, 512), (3, 130, 4096), (10, 96, 1024), (40, 300, 2048), (200, 260, 512)])
def test_mxfp8_wide_scales(M_, N, K):
    """E8M0 block scales over codes 100..160 (2^-27 .. 2^33) with every finite E4M3 code:
    each kernel (vector-ALU gemv, MFMA gemv, tiled GEMM) on the whole exponent spread."""
    inp = workloads.make_mxfp8(M_, N, K, seed=3, config_id=71, e8m0=(100, 160))
    say(f"mxfp8 wide scales M={M_} N={N} K={K}")
    got = _run_mxfp8(inp)
    _, ref, mass = omx.mxfp8_gemm(inp.x, inp.w, inp.s)
    check_band(band.classify(got, ref, mass), f"mxfp8 wide scales {M_}x{N}x{K}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M_", [1, 512])
def test_mxfp8_config(M_):
    inp = workloads.mxfp8_config(M_)
    say(f"mxfp8 config M={M_} N={inp.N} K={inp.K}")
    got = _run_mxfp8(inp)
    if M_ == 1:
        rows = np.arange(1)
    else:
        # the first and last row of every 128-row tile of the GEMM, and four more
        tiles = [r for t0 in range(0, M_, 128) for r in (t0, min(t0 + 128, M_) - 1)]
        rows = np.unique(np.concatenate([tiles, np.random.default_rng(3).choice(M_, 4, replace=False)]))
    _, ref, mass = omx.mxfp8_gemm(inp.x, inp.w, inp.s, rows=rows)
    check_band(band.classify(got[rows], ref, mass), f"mxfp8 config M={M_}", f"out ({rows.size} rows x {inp.N})")


# ---------------------------------------------------------------- routing in the FFN launch
@pytest.mark.parametrize("T,d,f,E,k", [(4, 2048, 768, 128, 8), (1, 32, 32, 1, 1), (3, 96, 64, 5, 2),
                                       (16, 160, 96, 6, 3), (8, 512, 256, 256, 16), (16, 256, 128, 200, 4),
                                       (2, 256, 128, 256, 16), (4, 256, 128, 160, 16), (3, 128, 64, 64, 4),
                                       (4, 128, 64, 65, 8), (5, 128, 64, 200, 13)])
def test_route_ffn_fused(T, d, f, E, k):
    """moe_route_expert_ffn_nvfp4 against the oracle (routing bit-exact, whole layer in the
    band) and against the separate moe_route_topk + moe_expert_ffn_nvfp4 calls (same bits).
    Shapes cover the launch's routing forms: one wave a token (T <= 4) with 1, 2 and 4 keys a
    lane (E <= 64, <= 128, <= 256), a 16-lane row a token (T > 4), and the row lists from one
    wave's ballots (T * k <= 64, 64 included) or from ranks, counts and a scan (T * k = 65)."""
    import torch
    import nvfp4_block_scaled_topk_amd as M
    inp = workloads.make_moe(T, d, f, E, k, seed=4, config_id=63, zipf=True)
    say(f"fused route+FFN T={T} d={d} f={f} E={E} k={k}")
    x, logits, ex = upload_moe(inp)
    (ids, w, off, sr, ro), y = M.route_expert_ffn_nvfp4(logits, x, ex, k)
    out = M.combine(y, ro, w)
    torch.cuda.synchronize()
    res = dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), offsets=off.cpu().numpy(), sorted_rows=sr.cpu().numpy(),
               row_of=ro.cpu().numpy(), y_rows=y.cpu().numpy(), out=out.view(torch.int16).cpu().numpy().view(np.uint16))
    check_layer_full(inp, res, f"fused T{T}E{E}k{k}")
    sep = run_moe(inp)
    for key in ("ids", "offsets", "sorted_rows", "row_of"):
        assert np.array_equal(res[key], sep[key]), key
    assert np.array_equal(res["w"].view(np.uint32), sep["w"].view(np.uint32))
    assert np.array_equal(res["y_rows"].view(np.uint32), sep["y_rows"].view(np.uint32))

