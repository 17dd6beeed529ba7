"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI (via the package binding), compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import nvfp4_block_scaled_topk_amd as M
from oracle import band, formats as F, moe


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# Every band check of a GPU test appends its counts here; the session writes them to a
# JSON file at its end (tests/conftest.py, MOE_PARITY_RECORDS).
RECORDS = []
# "explained" elements (outside the strict band, inside the slack) must stay rare: the
# slack covers bf16 rounding ties of h and fp32 sum-order effects, which touch well
# under one element in two hundred of these workloads
EXPLAINED_MAX = 0.005


# Measured errors that are reported, not bounded by the band (e.g. a lower-precision
# variant against the exact path); written beside the band records.
REPORTS = []


def check_band(rep, case, part="out"):
    """Record a band report and assert FAIL = 0 and explained <= 0.5 % of the elements."""
    RECORDS.append({"case": case, "part": part, "n": rep.n, "strict": rep.strict, "explained": rep.explained,
                    "fail": rep.fail, "worst_excess": rep.worst_excess})
    say(f"[{case}] {part}: {rep}")
    assert rep.ok(), f"{case} {part}: {rep}"
    assert rep.explained <= EXPLAINED_MAX * rep.n, f"{case} {part}: explained above 0.5 %: {rep}"
    return rep


def cover_tokens(offsets, sorted_rows, k, tile=128, skinny=32, rowset=16):
    """Tokens whose routed rows cover every grouped-GEMM tile and every weight-streaming
    expert of a prompt batch: for an expert with more than `skinny` rows, the first and
    last row of each `tile`-row tile; for the others, the first and last row of each of
    their `rowset`-row sets."""
    off = np.asarray(offsets, dtype=np.int64)
    rows = []
    for e in range(off.size - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        step = tile if b - a > skinny else rowset
        for t0 in range(a, b, step):
            rows += [t0, min(t0 + step, b) - 1]
    return np.unique(np.asarray(sorted_rows, dtype=np.int64)[np.asarray(rows)] // k)


def upload_moe(inp, device="cuda"):
    x = torch.from_numpy(inp.x.view(np.int16)).to(device).view(torch.bfloat16)
    logits = torch.from_numpy(inp.logits).to(device)
    ex = M.NVFP4Experts.from_numpy(inp, device)
    return x, logits, ex


def run_moe(inp, device="cuda", nan_canary=True):
    """Run route -> FFN -> combine on the GPU; returns numpy arrays."""
    x, logits, ex = upload_moe(inp, device)
    T, d, k = inp.T, inp.d, inp.k
    ids, w, off, srows, rof = M.route_topk(logits, k)
    y_rows = torch.full((T * k, d), float("nan"), dtype=torch.float32, device=device) if nan_canary else None
    y_rows = M.expert_ffn_nvfp4(x, ex, off, srows, k, out=y_rows)
    out = M.combine(y_rows, rof, w)
    torch.cuda.synchronize()
    res = dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), offsets=off.cpu().numpy(),
               sorted_rows=srows.cpu().numpy(), row_of=rof.cpu().numpy(),
               y_rows=y_rows.cpu().numpy(), out=out.view(torch.int16).cpu().numpy().view(np.uint16))
    return res


def weight_tolerance(logits_sel, w64, k):
    """Bound on |w_gpu - w| for the fp32 softmax of the selected logits: the
    exponential and the division each within a couple of ulps, the k-term sum
    within k ulps, relative to each weight; plus a tiny absolute floor."""
    return (6 + k) * 2.0 ** -24 * np.abs(w64) + 2.0 ** -40


def check_routing(inp, res, where=""):
    ids, w = moe.route(inp.logits, inp.k)
    rl = moe.row_lists(ids, inp.E)
    assert np.array_equal(res["ids"], ids), f"{where}: top-k ids differ"
    assert np.array_equal(res["offsets"], rl.offsets), f"{where}: expert offsets differ"
    assert np.array_equal(res["sorted_rows"], rl.sorted_rows), f"{where}: sorted_rows differ"
    assert np.array_equal(res["row_of"], rl.row_of), f"{where}: row_of differ"
    tol = weight_tolerance(None, w, inp.k)
    err = np.abs(res["w"].astype(np.float64) - w)
    assert np.all(err <= tol), f"{where}: weights max err {err.max():.3g}"
    assert np.all(np.abs(res["w"].astype(np.float64).sum(axis=1) - 1.0) <= inp.k * 2.0 ** -22)
    return ids, w, rl


def check_layer_full(inp, res, where=""):
    """Whole-layer parity (every row, every output element)."""
    check_routing(inp, res, where)
    ref = moe.moe_layer(inp)
    assert not np.any(np.isnan(res["y_rows"])), f"{where}: unwritten expert rows (NaN canary)"
    check_band(band.classify_f32(res["y_rows"], ref.ffn.y_rows, ref.ffn.mass_y, ref.ffn.slack_h), where, "y_rows")
    return check_band(band.classify(res["out"], ref.out_bits, ref.mass, ref.slack), where, "out")


def check_layer_sampled(inp, res, tokens, where="", threads=8):
    """Parity on sampled tokens (all of their k rows and d outputs). The oracle's experts
    are independent and run on `threads` threads."""
    from concurrent.futures import ThreadPoolExecutor

    ids, w, rl = check_routing(inp, res, where)
    assert not np.any(np.isnan(res["y_rows"])), f"{where}: unwritten expert rows (NaN canary)"
    say(f"[{where}] oracle for {len(tokens)} sampled tokens")
    with ThreadPoolExecutor(threads) as ex:
        def progress_map(fn, items):
            for i, r in enumerate(ex.map(fn, items)):
                if i % 16 == 15:
                    say(f"[{where}] oracle: {i + 1} of {len(items)} experts")
                yield r
        ref = moe.moe_tokens(inp, tokens, ids=ids, w=w, rl=rl, map_fn=progress_map)
    rows = ref.ffn.rows
    check_band(band.classify_f32(res["y_rows"][rows], ref.ffn.y_rows, ref.ffn.mass_y, ref.ffn.slack_h),
               where, f"y_rows ({rows.size} sampled rows)")
    return check_band(band.classify(res["out"][np.asarray(tokens)], ref.out_bits, ref.mass, ref.slack),
                      where, f"out ({len(tokens)} sampled tokens)")
