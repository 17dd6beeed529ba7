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
    rep_rows = band.classify_f32(res["y_rows"], ref.ffn.y_rows, ref.ffn.mass_y, ref.ffn.slack_h)
    rep_out = band.classify(res["out"], ref.out_bits, ref.mass, ref.slack)
    say(f"[{where}] y_rows: {rep_rows}")
    say(f"[{where}] out:    {rep_out}")
    assert rep_rows.ok(), f"{where}: y_rows {rep_rows}"
    assert rep_out.ok(), f"{where}: out {rep_out}"
    return rep_out


def check_layer_sampled(inp, res, tokens, where=""):
    """Parity on sampled tokens (all of their k rows and d outputs)."""
    ids, w, rl = check_routing(inp, res, where)
    assert not np.any(np.isnan(res["y_rows"])), f"{where}: unwritten expert rows (NaN canary)"
    ref = moe.moe_tokens(inp, tokens, ids=ids, w=w, rl=rl)
    rows = ref.ffn.rows
    rep_rows = band.classify_f32(res["y_rows"][rows], ref.ffn.y_rows, ref.ffn.mass_y, ref.ffn.slack_h)
    rep_out = band.classify(res["out"][np.asarray(tokens)], ref.out_bits, ref.mass, ref.slack)
    say(f"[{where}] sampled {len(tokens)} tokens; y_rows: {rep_rows}")
    say(f"[{where}] sampled out: {rep_out}")
    assert rep_rows.ok(), f"{where}: y_rows {rep_rows}"
    assert rep_out.ok(), f"{where}: out {rep_out}"
    return rep_out
