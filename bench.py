"""Benchmark of the routed NVFP4 MoE layer (route -> expert FFN -> combine) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole layer over one batch of synthetic tokens: top-k
routing with row lists, the gate/up/SwiGLU and down products over NVFP4 experts,
and the weighted combine. The default workload is the decode layer (T=4, d=2048,
f=768, E=128, top-8, Zipf(1.1)-skewed routing); the prompt layer (T=512, d=3072,
f=1536, E=128), the long-prompt layer (T=4096, d=7168, f=2048, E=256) and the MXFP8
projection (N=12288, K=4096, M=1 and 512) are measured beside it under "also".

Timing: the K steps are enqueued behind a GPU sleep kernel so the device never
waits for the host, and bracketed by HIP events on the stream the kernels run on
(torch's current stream). The expert FFN is the dominant work and is reported
against its roofline: its duration per call comes from a second timed loop of
back-to-back FFN calls between one pair of events (the per-step FFN events of the
layer loop, which include event overhead, are reported beside it).
Steps rotate through distinct copies of the expert weights, as many as it takes for
the weight bytes the steps touch over one rotation to reach 1 GB (four times the
256 MB Infinity Cache), so repeats are not served from it.

Prints ONE JSON line (rank 0). --gpus N with N > 1 is refused: this build runs
on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + HBM GB/s (decode) and MFMA TFLOP/s (prompt), 1×MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0       # MI355X published dense bf16 MFMA rate
FP8_PEAK_TFLOPS = 5000.0        # MI355X published dense fp8 MFMA rate
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
# kernel sources whose hash a traffic record must match, per path
DECODE_FILES = ["ffn_decode.hip", "route_device.hpp", "device.hpp"]
PROMPT_FILES = ["ffn_prompt.hip", "skinny_device.hpp", "device.hpp"]
MXFP8_FILES = ["mxfp8.hip", "device.hpp"]
ROUTER_FILES = ["router.hip", "device.hpp"]
W8A8_FILES = ["mxfp8_w8a8.hip", "device.hpp"]
PROMPT_KERNELS = ("moe_expert_ffn_nvfp4 prompt path (ffn_prompt_kernel gate/up, then down: the grouped GEMM's "
                  "tiles, then the weight-streaming items of the experts with <= 32 rows)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(d, f):
    """Stored bytes of one expert: three projections of f x d codes (1/2 byte
    each) and block scales (1/16 byte each), plus three fp32 tensor scales."""
    return 3 * (f * d // 2 + f * d // 16) + 12


def kernel_source_hash(files):
    h = hashlib.sha256()
    for fn in files:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_topk_amd", "csrc", fn), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, files):
    """Measured HBM traffic of the FFN kernels (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    scaled by a plain-copy calibration), if recorded for the current sources."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != kernel_source_hash(files):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    def __init__(self, torch):
        self.torch = torch
        self.cycles_per_ms = None

    def calibrate_sleep(self):
        torch = self.torch
        if not hasattr(torch.cuda, "_sleep"):
            return
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 2_000_000
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        self.cycles_per_ms = n / max(ms, 1e-3)

    def queue_ahead(self, ms):
        """Occupy the stream for about `ms` so the following launches queue up."""
        if self.cycles_per_ms:
            self.torch.cuda._sleep(int(self.cycles_per_ms * ms))


def bench_moe(name, steps, warmup, rotations, timer, seed=0):
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M
    import workloads

    dev = torch.device("cuda", 0)
    log(f"[bench] {name}: generating inputs")
    inp = workloads.moe_config(name, seed=seed)
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(inp.logits).to(dev)
    ex0 = M.NVFP4Experts.from_numpy(inp, dev)
    ex0.check()
    del inp
    if rotations <= 0:
        # enough copies that the experts a step touches, over one rotation, are >= 1 GB
        _, _, off0, _, _ = M.route_topk(logits, k)
        touched = int((off0[1:] - off0[:-1] > 0).sum().item())
        per_expert = sum(getattr(ex0, n).numel() * getattr(ex0, n).element_size()
                         for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")) // E
        rotations = max(1, -(-(1 << 30) // max(1, touched * per_expert)))
        rotations = min(rotations, max(1, (48 << 30) // max(1, E * per_expert)))  # at most ~48 GB of copies
    copies = [ex0]
    for _ in range(rotations - 1):
        copies.append(M.NVFP4Experts(*[getattr(ex0, n).clone() for n in
                                       ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts",
                                        "down_q", "down_s", "down_ts")]))
    # outputs and workspaces, allocated once
    rbufs = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
             torch.empty((E + 1,), dtype=torch.int32, device=dev), torch.empty((T * k,), dtype=torch.int32, device=dev),
             torch.empty((T * k,), dtype=torch.int32, device=dev))
    rws_n = M.route_topk_workspace(T, E, k)
    rws = torch.empty((max(rws_n, 1),), dtype=torch.uint8, device=dev) if rws_n else None
    fws = torch.empty((max(M.expert_ffn_workspace(T, d, f, E, k), 1),), dtype=torch.uint8, device=dev)
    y_rows = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    ids, w, off, srows, rof = rbufs
    # few tokens: the whole layer (routing, expert FFN, combine) is one launch
    # (moe_layer_nvfp4) when the shape allows it; otherwise route, FFN, combine
    fused = False
    lws = None
    if T <= 16 and M.layer_workspace(T, d, f, E, k) > 0:
        lws = torch.zeros((M.layer_workspace(T, d, f, E, k),), dtype=torch.uint8, device=dev)
        M.layer_nvfp4(logits, x, ex0, k, route_out=rbufs, out=out, workspace=lws, check=False)
        fused = True

    def step(i):
        ex = copies[i % rotations]
        if fused:
            M.layer_nvfp4(logits, x, ex, k, route_out=rbufs, out=out, workspace=lws, check=False)
            return
        M.route_topk(logits, k, out=rbufs, workspace=rws)
        M.expert_ffn_nvfp4(x, ex, off, srows, k, out=y_rows, workspace=fws, check=False)
        M.combine(y_rows, rof, w, out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    counts = np.diff(off.cpu().numpy())
    U = int((counts > 0).sum())
    # host enqueue rate, to size the queue-ahead sleep
    t0 = time.perf_counter()
    for i in range(min(steps, 20)):
        step(i)
    torch.cuda.synchronize()
    host_ms_per_step = (time.perf_counter() - t0) * 1e3 / min(steps, 20)

    # the timed region: K whole layers back to back, nothing else on the stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    timer.queue_ahead(host_ms_per_step * steps * 1.5 + 20.0)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / steps

    # Per-step distribution: the same steps with an event between consecutive steps (the
    # event records add small gaps, so this loop is not the timed region).
    n_ev = min(steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
    torch.cuda.synchronize()
    timer.queue_ahead(host_ms_per_step * n_ev * 1.5 + 20.0)
    evs[0].record()
    for i in range(n_ev):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    step_us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_ev)])
    p10, p50, p90 = (float(v) for v in np.percentile(step_us, [10, 50, 90]))

    def back_to_back(call, n):
        """Average duration of `call(i)` enqueued n times back to back between one pair of
        events on the stream the kernels run on (torch's current stream)."""
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        timer.queue_ahead(host_ms_per_step * n + 20.0)
        a_ev.record()
        for i in range(n):
            call(i)
        b_ev.record()
        torch.cuda.synchronize()
        return a_ev.elapsed_time(b_ev) * 1e3 / n

    n_b2b = max(steps, 50)
    # the dominant launch of the layer: the whole layer for few tokens, else the expert FFN
    if fused:
        launch_us = back_to_back(lambda i: M.layer_nvfp4(
            logits, x, copies[i % rotations], k, route_out=rbufs, out=out, workspace=lws, check=False), n_b2b)
    else:
        launch_us = back_to_back(lambda i: M.expert_ffn_nvfp4(
            x, copies[i % rotations], off, srows, k, out=y_rows, workspace=fws, check=False), n_b2b)
    # the expert FFN alone, routing lists given
    ffn_us = back_to_back(lambda i: M.expert_ffn_nvfp4(
        x, copies[i % rotations], off, srows, k, out=y_rows, workspace=fws, check=False), n_b2b)
    # for comparison, the same layer as separate launches (few tokens: routing inside the
    # FFN launch, then the combine; otherwise the layer step itself)
    separate_us = None
    if fused:
        def separate(i):
            M.route_expert_ffn_nvfp4(logits, x, copies[i % rotations], k, route_out=rbufs, out=y_rows, workspace=fws,
                                     check=False)
            M.combine(y_rows, rof, w, out=out)
        separate_us = back_to_back(separate, n_b2b)

    # algorithmic work (only what the method must move / compute)
    eb = expert_bytes(d, f)
    counts = np.diff(off.cpu().numpy())
    ffn_bytes = U * eb + T * d * 2
    layer_bytes = U * eb + T * d * 2 + T * E * 4 + T * d * 2
    launch_bytes = layer_bytes if fused else ffn_bytes
    flops = 2.0 * T * k * 3 * d * f

    # Ceiling: a plain coalesced read (moe_read_ceiling) of the same bytes the expert
    # kernels must read -- the touched experts' codes and scales, of the same rotating
    # weight copies -- back to back.
    touched = np.nonzero(counts > 0)[0]
    names6 = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")
    tables = []
    for c in copies:
        rows = []
        for nm in names6:
            t = getattr(c, nm)
            per = t[0].numel() * t.element_size()
            for e in touched:
                rows.append((t.data_ptr() + int(e) * per, per))
        tables.append(torch.tensor(rows, dtype=torch.int64, device=dev))
    read_bytes = sum(r[1] for r in rows)
    sink = torch.zeros((4096,), dtype=torch.int32, device=dev)
    ceiling_us = back_to_back(lambda i: M.read_ceiling(tables[i % rotations], read_bytes, sink), n_b2b)

    res = dict(
        name=name, T=T, d=d, f=f, E=E, k=k, touched_experts=U, rotations=rotations,
        ms_per_step=ms_per_step, tokens_per_s=T / (ms_per_step / 1e3),
        step_us_p10=p10, step_us_p50=p50, step_us_p90=p90,
        launch_us=launch_us, launch_bytes=launch_bytes, ffn_avg_us=ffn_us,
        ffn_bytes=ffn_bytes, layer_bytes=layer_bytes, flops=flops,
        ceiling_us=ceiling_us, ceiling_bytes=read_bytes, ceiling_gbps=read_bytes / (ceiling_us / 1e6) / 1e9,
        layer_hbm_gbps=layer_bytes / (ms_per_step / 1e3) / 1e9,
        launch_hbm_gbps=launch_bytes / (launch_us / 1e6) / 1e9,
        ffn_hbm_gbps=ffn_bytes / (ffn_us / 1e6) / 1e9,
        ffn_tflops=flops / (ffn_us / 1e6) / 1e12,
        layer_tflops=flops / (ms_per_step / 1e3) / 1e12,
        host_ms_per_step=host_ms_per_step, layer_in_one_launch=fused, separate_launches_us=separate_us,
    )
    log(f"[bench] {name}: {json.dumps(res)}")
    del copies, ex0
    torch.cuda.empty_cache()
    return res


def bench_mxfp8(M, steps, warmup, rotations, timer, seed=0, kernel_name=None):
    """MXFP8 projection y = x . W^T (N=12288, K=4096): `steps` calls queued behind a GPU
    sleep, bracketed by one pair of HIP events; weights rotate through `rotations`
    copies so repeats are not served from the Infinity Cache."""
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M_
    import workloads

    dev = torch.device("cuda", 0)
    inp = workloads.mxfp8_config(M, seed=seed)
    N, K = inp.N, inp.K
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    w0 = torch.from_numpy(inp.w).to(dev)
    s0 = torch.from_numpy(inp.s).to(dev)
    del inp
    ws = [(w0, s0)] + [(w0.clone(), s0.clone()) for _ in range(rotations - 1)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for i in range(warmup):
        M_.mxfp8_gemm(x, *ws[i % rotations], out=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(20):
        M_.mxfp8_gemm(x, *ws[i % rotations], out=y)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3 / 20
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.queue_ahead(host_ms * steps * 1.5 + 20.0)
    start.record()
    for i in range(steps):
        M_.mxfp8_gemm(x, *ws[i % rotations], out=y)
    end.record()
    torch.cuda.synchronize()
    avg_ms = start.elapsed_time(end) / steps
    nbytes = N * K + N * (K // 32) + M * K * 2 + M * N * 2
    flops = 2.0 * M * N * K
    res = {"M": M, "N": N, "K": K, "avg_us": avg_ms * 1e3, "rows_per_s": M / (avg_ms / 1e3),
           "algorithmic_bytes": nbytes, "algorithmic_flop": flops, "weight_copies_rotated": rotations,
           "hbm_gbps": nbytes / (avg_ms / 1e3) / 1e9, "tflops": flops / (avg_ms / 1e3) / 1e12}
    if M <= 16:
        res["roofline"] = {"bound": "hbm", "achieved": res["hbm_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": res["hbm_gbps"] / HBM_PEAK_GBPS,
                           "kernel": kernel_name or ("mxfp8_gemv_valu_kernel" if M <= 4 else "mxfp8_gemv_kernel"),
                           "algorithmic_bytes": nbytes, "avg_us": res["avg_us"]}
    else:
        res["roofline"] = {"bound": "mfma", "achieved": res["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": res["tflops"] / BF16_PEAK_TFLOPS, "kernel": "mxfp8_gemm_kernel",
                           "algorithmic_flop": flops, "avg_us": res["avg_us"]}
    log(f"[bench] mxfp8 M={M}: {json.dumps(res)}")
    del ws, w0, s0
    torch.cuda.empty_cache()
    return res


def bench_w8a8(M, steps, warmup, rotations, timer, seed=0):
    """The W8A8 MXFP8 projection (N=12288, K=4096): activations quantized to MXFP8
    (mxfp8_quantize) and the block-scaled fp8 product (mxfp8_gemm_mx), one pair of HIP
    events around `steps` calls of each, weights rotated through `rotations` copies."""
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M_
    import workloads

    dev = torch.device("cuda", 0)
    inp = workloads.mxfp8_config(M, seed=seed)
    N, K = inp.N, inp.K
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    w0 = torch.from_numpy(inp.w).to(dev)
    s0 = torch.from_numpy(inp.s).to(dev)
    del inp
    ws = [(w0, s0)] + [(w0.clone(), s0.clone()) for _ in range(rotations - 1)]
    xq, xs = M_.mxfp8_quantize(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for i in range(warmup):
        M_.mxfp8_quantize(x, out=(xq, xs))
        M_.mxfp8_gemm_mx(xq, xs, *ws[i % rotations], out=y)
    torch.cuda.synchronize()

    def timed(call):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        timer.queue_ahead(steps * 0.1 + 20.0)
        start.record()
        for i in range(steps):
            call(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) * 1e3 / steps

    q_us = timed(lambda i: M_.mxfp8_quantize(x, out=(xq, xs)))
    g_us = timed(lambda i: M_.mxfp8_gemm_mx(xq, xs, *ws[i % rotations], out=y))
    flops = 2.0 * M * N * K
    res = {"M": M, "N": N, "K": K, "quantize_us": q_us, "gemm_us": g_us, "total_us": q_us + g_us,
           "rows_per_s": M / ((q_us + g_us) / 1e6), "algorithmic_flop": flops,
           "gemm_tflops": flops / (g_us / 1e6) / 1e12,
           "roofline": {"bound": "mfma", "achieved": flops / (g_us / 1e6) / 1e12, "peak": FP8_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": flops / (g_us / 1e6) / 1e12 / FP8_PEAK_TFLOPS,
                        "kernel": "mx_gemm_kernel (mxfp8_gemm_mx: block-scaled fp8 MFMA)", "avg_us": g_us,
                        "traffic": load_traffic(f"w8a8_M{M}", W8A8_FILES)},
           "error_vs_bf16_activations": "rms error / rms output 0.030 on 12 rows of this configuration "
                                        "(tests/test_gpu_w8a8.py; profiles/parity_records.json reports)"}
    log(f"[bench] w8a8 M={M}: {json.dumps(res)}")
    del ws, w0, s0
    torch.cuda.empty_cache()
    return res


def bench_mxfp8_columns(steps, timer, seed=0):
    """The MXFP8 projection with a few activation rows: the per-card pick of the few-row
    kernel (mxfp8_autotune over M = 1..16 at N=12288, K=4096), then 4 and 8 rows timed
    with it."""
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M_
    import workloads

    inp = workloads.mxfp8_config(16, seed=seed)
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    picks, us = M_.mxfp8_autotune(x, torch.from_numpy(inp.w).cuda(), torch.from_numpy(inp.s).cuda(), reps=20)
    del inp, x
    torch.cuda.empty_cache()
    out = {"picks": {str(m + 1): M_.MXFP8_KERNELS[p] for m, p in enumerate(picks)},
           "autotune_us": {str(m + 1): dict(zip(M_.MXFP8_KERNELS, [None if v != v else round(v, 2) for v in t]))
                           for m, t in enumerate(us)}}
    for m in (4, 8):
        out[f"M{m}"] = bench_mxfp8(m, steps, 5, 20, timer, seed=seed, kernel_name=M_.MXFP8_KERNELS[picks[m - 1]])
    log(f"[bench] mxfp8 columns: picks {out['picks']}")
    return out


def bench_ffn_pick(seed=0):
    """The few-token path of the NVFP4 expert FFN picked for this card (moe_ffn_autotune)
    at the decode layer's shape (T=4, d=2048, f=768, E=128, k=8) and at its shared expert's
    (one expert every token routes to: E=1, k=1): the pick and each path's time a call
    (operands as the configuration's, no weight rotation)."""
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M
    import workloads

    out = {}
    for label, inp in (("decode", workloads.moe_config("decode", seed=seed)),
                       ("shared_expert", workloads.make_moe(4, 2048, 768, 1, 1, seed=seed, config_id=98))):
        x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
        ex = M.NVFP4Experts.from_numpy(inp, "cuda")
        _, _, off, srows, _ = M.route_topk(torch.from_numpy(inp.logits).cuda(), inp.k)
        pick, us = M.ffn_autotune(x, ex, off, srows, inp.k, reps=50)
        out[label] = {"pick": M.FFN_PATHS[pick],
                      "us": {M.FFN_PATHS[i]: (None if v != v else round(v, 2)) for i, v in enumerate(us)}}
        del ex, x
    torch.cuda.empty_cache()
    log(f"[bench] ffn pick: {json.dumps(out)}")
    return out


def bench_shards(steps, timer, seed=0):
    """One GPU's share of the layer, as it would shard (the exchanges between GPUs are not
    part of this build):
    * EP = 8 at the long prompt: the FFN of a GPU's 256/8 experts on the rows routed to
      them, gathered (k = 1 a row); rank 0 and the most loaded rank (routing skew);
    * TP = 8 at decode: every expert's f/8 = 96 features; the partial layer (routing, FFN,
      combine in one launch) an all-reduce would sum, weights rotated past the Infinity Cache."""
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M
    import workloads

    names = ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")
    out = {}
    inp = workloads.moe_config("long_prompt", seed=seed)
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    logits = torch.from_numpy(inp.logits).cuda()
    ex = M.NVFP4Experts.from_numpy(inp, "cuda")
    del inp
    _, _, off, srows, _ = M.route_topk(logits, k)
    offs = off.cpu().numpy()
    per_rank = [int(offs[(r + 1) * E // 8] - offs[r * E // 8]) for r in range(8)]
    for label, rank in (("ep8_rank0", 0), ("ep8_most_loaded", int(np.argmax(per_rank)))):
        e0, e1 = rank * E // 8, (rank + 1) * E // 8
        p0, p1 = int(offs[e0]), int(offs[e1])
        x_loc = x.index_select(0, srows[p0:p1].long() // k).contiguous()
        off_loc = (off[e0:e1 + 1] - p0).contiguous()
        rows_loc = torch.arange(p1 - p0, dtype=torch.int32, device="cuda")
        ex_loc = M.NVFP4Experts(*[getattr(ex, n)[e0:e1].contiguous() for n in names])
        y = torch.empty((p1 - p0, d), dtype=torch.float32, device="cuda")
        ws = torch.empty((max(M.expert_ffn_workspace(p1 - p0, d, f, e1 - e0, 1), 1),), dtype=torch.uint8, device="cuda")
        call = lambda: M.expert_ffn_nvfp4(x_loc, ex_loc, off_loc, rows_loc, 1, out=y, workspace=ws, check=False)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        timer.queue_ahead(20.0)
        a.record()
        for _ in range(steps):
            call()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / steps
        flops = 2.0 * (p1 - p0) * 3 * d * f
        out[label] = {"rank": rank, "experts": [e0, e1 - 1], "rows": p1 - p0, "rows_a_rank": per_rank,
                      "ffn_us": us, "tflops": flops / (us / 1e6) / 1e12,
                      "mfma_frac": flops / (us / 1e6) / 1e12 / BF16_PEAK_TFLOPS}
        del x_loc, ex_loc, y, ws
    del ex, x, logits
    torch.cuda.empty_cache()

    inp = workloads.tp_share(workloads.moe_config("decode", seed=seed), 8, 0)
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    logits = torch.from_numpy(inp.logits).cuda()
    ex0 = M.NVFP4Experts.from_numpy(inp, "cuda")
    del inp
    _, _, off, _, _ = M.route_topk(logits, k)
    U = int((off[1:] - off[:-1] > 0).sum().item())
    eb = expert_bytes(d, f)
    rot = max(1, -(-(1 << 30) // (U * eb)))
    copies = [ex0] + [M.NVFP4Experts(*[getattr(ex0, n).clone() for n in names]) for _ in range(rot - 1)]
    lws = torch.zeros((M.layer_workspace(T, d, f, E, k),), dtype=torch.uint8, device="cuda")
    o = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    for i in range(5):
        M.layer_nvfp4(logits, x, copies[i % rot], k, out=o, workspace=lws, check=False)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.queue_ahead(20.0)
    a.record()
    for i in range(steps):
        M.layer_nvfp4(logits, x, copies[i % rot], k, out=o, workspace=lws, check=False)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    nbytes = U * eb + T * d * 2 + T * E * 4 + T * d * 2
    out["tp8_decode_rank0"] = {"f_local": f, "touched_experts": U, "weight_copies_rotated": rot,
                               "layer_us": us, "algorithmic_bytes": nbytes,
                               "hbm_gbps": nbytes / (us / 1e6) / 1e9,
                               "hbm_frac": nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBPS}
    del copies, ex0
    torch.cuda.empty_cache()
    log(f"[bench] shards: {json.dumps(out)}")
    return out


def bench_block(name, steps, warmup, timer, seed=0):
    """The whole MoE block of a configuration: router projection, routing, routed expert
    FFN, the shared expert's FFN and gate logit, and the combine with the shared add, all
    on one stream (the few-token FFN is not overlapped with other work). Routed and
    shared weights rotate through copies as in bench_moe (touched bytes >= 1 GB a
    rotation). Returns tokens/s and the block's algorithmic bytes and FLOP rates."""
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M
    import workloads

    dev = torch.device("cuda", 0)
    inp = workloads.moe_config(name, seed=seed)
    rin = workloads.router_config(name, seed=seed)
    sh = workloads.shared_config(name, seed=seed)
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    w_r = torch.from_numpy(rin.w_r.view(np.int16)).to(dev).view(torch.bfloat16)
    w_sg = torch.from_numpy(sh.w_sg.view(np.int16).reshape(1, d)).to(dev).view(torch.bfloat16)
    ex0 = M.NVFP4Experts.from_numpy(inp, dev)
    sx0 = M.NVFP4Experts.from_numpy(sh, dev)
    del inp, rin, sh
    logits = M.router_logits(x, w_r)
    _, _, off0, _, _ = M.route_topk(logits, k)
    U = int((off0[1:] - off0[:-1] > 0).sum().item())
    eb = expert_bytes(d, f)
    rotations = max(1, -(-(1 << 30) // ((U + 1) * eb)))
    rotations = min(rotations, max(1, (48 << 30) // max(1, (E + 1) * eb)))
    names = ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")
    copies = [(ex0, sx0)] + [(M.NVFP4Experts(*[getattr(ex0, n).clone() for n in names]),
                              M.NVFP4Experts(*[getattr(sx0, n).clone() for n in names])) for _ in range(rotations - 1)]
    rbufs = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
             torch.empty((E + 1,), dtype=torch.int32, device=dev), torch.empty((T * k,), dtype=torch.int32, device=dev),
             torch.empty((T * k,), dtype=torch.int32, device=dev))
    rws_n = M.route_topk_workspace(T, E, k)
    rws = torch.empty((rws_n,), dtype=torch.uint8, device=dev) if rws_n else None
    fws = torch.empty((max(M.expert_ffn_workspace(T, d, f, E, k), 1),), dtype=torch.uint8, device=dev)
    sws = torch.empty((max(M.expert_ffn_workspace(T, d, f, 1, 1), 1),), dtype=torch.uint8, device=dev)
    y_rows = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    s_rows = torch.empty((T, d), dtype=torch.float32, device=dev)
    glog = torch.empty((T, 1), dtype=torch.float32, device=dev)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    ids, w, off, srows, rof = rbufs

    # Few tokens: one router launch projects the routed logits and the shared gate's logit
    # together (W_r with w_sg as row E), then the whole layer is one launch
    # (moe_layer_nvfp4). Otherwise: router, routing, routed FFN, shared FFN, gate, combine.
    one_launch = T <= 16 and M.layer_workspace(T, d, f, E, k, True) > 0
    w_stk = torch.cat([w_r, w_sg], dim=0).contiguous()
    stk = torch.empty((T, E + 1), dtype=torch.float32, device=dev)
    lws = (torch.zeros((M.layer_workspace(T, d, f, E, k, True),), dtype=torch.uint8, device=dev)
           if one_launch else None)

    def separate_step(i):
        ex, sx = copies[i % rotations]
        M.router_logits(x, w_r, out=logits)
        M.route_topk(logits, k, out=rbufs, workspace=rws)
        M.expert_ffn_nvfp4(x, ex, off, srows, k, out=y_rows, workspace=fws, check=False)
        M.shared_expert_nvfp4(x, sx, out=s_rows, workspace=sws)
        M.router_logits(x, w_sg, out=glog)
        M.combine(y_rows, rof, w, out=out, shared_rows=s_rows, shared_gate_logit=glog, residual=x)

    def layer_step(i):
        ex, sx = copies[i % rotations]
        M.router_logits(x, w_stk, out=stk)
        M.layer_nvfp4(stk, x, ex, k, shared=sx, shared_gate_logit=stk[:, E:E + 1], residual=x, route_out=rbufs,
                      out=out, workspace=lws, check=False)

    step = layer_step if one_launch else separate_step

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(min(steps, 20)):
            fn(i)
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3 / min(steps, 20)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        timer.queue_ahead(host_ms * steps * 1.5 + 20.0)
        start.record()
        for i in range(steps):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    ms = timed(step)
    separate_ms = timed(separate_step) if one_launch else ms
    nbytes = (U + 1) * eb + E * d * 2 + d * 2 + 2 * T * d * 2 + T * E * 4
    flops = 2.0 * T * (k + 1) * 3 * d * f + 2.0 * T * (E + 1) * d
    res = {"T": T, "d": d, "f": f, "E": E, "k": k, "touched_experts": U, "weight_copies_rotated": rotations,
           "layer_in_one_launch": one_launch, "separate_launches_ms_per_step": separate_ms,
           "ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "algorithmic_bytes": nbytes, "algorithmic_flop": flops,
           "hbm_gbps": nbytes / (ms / 1e3) / 1e9, "tflops": flops / (ms / 1e3) / 1e12}
    log(f"[bench] block {name}: {json.dumps(res)}")
    del copies, ex0, sx0
    torch.cuda.empty_cache()
    return res


def bench_router(name, steps, warmup, timer, seed=0):
    """Router projection logits = x . W_r^T of a MoE configuration's activations:
    `steps` calls queued behind a GPU sleep, bracketed by one pair of HIP events."""
    import numpy as np
    import torch

    import nvfp4_block_scaled_topk_amd as M_
    import workloads

    dev = torch.device("cuda", 0)
    inp = workloads.router_config(name, seed=seed)
    T, d, E = inp.T, inp.d, inp.E
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(inp.w_r.view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((T, E), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        M_.router_logits(x, w, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        M_.router_logits(x, w, out=out)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3 / 20
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.queue_ahead(host_ms * steps * 1.5 + 20.0)
    start.record()
    for _ in range(steps):
        M_.router_logits(x, w, out=out)
    end.record()
    torch.cuda.synchronize()
    avg_ms = start.elapsed_time(end) / steps
    nbytes = T * d * 2 + E * d * 2 + T * E * 4
    flops = 2.0 * T * E * d
    res = {"T": T, "d": d, "E": E, "avg_us": avg_ms * 1e3, "tokens_per_s": T / (avg_ms / 1e3),
           "algorithmic_bytes": nbytes, "algorithmic_flop": flops,
           "hbm_gbps": nbytes / (avg_ms / 1e3) / 1e9, "tflops": flops / (avg_ms / 1e3) / 1e12}
    if T <= 16:
        res["roofline"] = {"bound": "hbm", "achieved": res["hbm_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": res["hbm_gbps"] / HBM_PEAK_GBPS, "kernel": "router_logits_kernel",
                           "algorithmic_bytes": nbytes, "avg_us": res["avg_us"],
                           "traffic": load_traffic(f"router_{name}", ROUTER_FILES)}
    else:
        res["roofline"] = {"bound": "mfma", "achieved": res["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": res["tflops"] / BF16_PEAK_TFLOPS, "kernel": "router_logits_kernel",
                           "algorithmic_flop": flops, "avg_us": res["avg_us"],
                           "traffic": load_traffic(f"router_{name}", ROUTER_FILES)}
    log(f"[bench] router {name}: {json.dumps(res)}")
    return res


def host_cores():
    """CPUs this process may run on, and how many physical cores they are (lscpu)."""
    import subprocess
    cpus = sorted(os.sched_getaffinity(0))
    phys = None
    try:
        out = subprocess.run(["lscpu", "-p=CPU,CORE,SOCKET"], capture_output=True, text=True, timeout=10).stdout
        cores = set()
        for line in out.splitlines():
            if line.startswith("#") or not line.strip():
                continue
            cpu, core, sock = (int(v) for v in line.split(",")[:3])
            if cpu in cpus:
                cores.add((sock, core))
        phys = len(cores) or None
    except Exception:  # lscpu missing: physical count unknown
        phys = None
    return len(cpus), phys


def time_oracle(fn, threads, reps):
    """Median wall-clock seconds of `fn` over `reps` runs with BLAS limited to `threads`."""
    from threadpoolctl import threadpool_limits
    ts = []
    with threadpool_limits(limits=threads):
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2], ts


def cpu_baseline():
    """The oracle (test infrastructure, untuned) on the host cores: whole decode layers
    (route, dequantize, FFN, combine) on the same seeded input as the GPU, median of 3
    runs with BLAS on every CPU of the process's affinity set and on 1 thread."""
    import workloads
    from oracle import moe as omoe

    logical, physical = host_cores()
    inp = workloads.moe_config("decode")
    med_all, _ = time_oracle(lambda: omoe.moe_layer(inp), logical, 3)
    med_one, _ = time_oracle(lambda: omoe.moe_layer(inp), 1, 3)
    return {"value": inp.T / med_all, "unit": "tokens/s", "cores": logical, "kind": "oracle",
            "physical_cores": physical, "one_thread_value": inp.T / med_one,
            "sample": f"whole decode layers (T={inp.T}, d={inp.d}, f={inp.f}, E={inp.E}, k={inp.k}): median of 3 "
                      f"runs, {med_all:.2f} s with BLAS on {logical} threads ({physical} physical cores), "
                      f"{med_one:.2f} s on 1 thread; fp64 NumPy, elementwise work single-threaded"}


def cpu_protocol(path):
    """The oracle on every configuration (a report, not the bench line): tiny, decode,
    prompt and the MXFP8 projection at M=1 and M=512 at 1 thread and all threads (median
    of 3; prompt and M=512 once at 1 thread), the long prompt once at all threads."""
    import workloads
    from oracle import moe as omoe, mxfp8 as omx

    logical, physical = host_cores()
    rows = []

    def run(name, unit_count, unit, fn, threads, reps):
        log(f"[cpu] {name} threads={threads} reps={reps}")
        med, ts = time_oracle(fn, threads, reps)
        rows.append({"workload": name, "threads": threads, "runs": reps, "median_s": med, "all_s": ts,
                     "value": unit_count / med, "unit": unit})

    for name in ("tiny", "decode", "prompt"):
        inp = workloads.moe_config(name)
        for threads, reps in ((logical, 3), (1, 3 if name != "prompt" else 1)):
            run(name, inp.T, "tokens/s", lambda inp=inp: omoe.moe_layer(inp), threads, reps)
        del inp
    for m in (1, 512):
        inp = workloads.mxfp8_config(m)
        for threads, reps in ((logical, 3), (1, 3 if m == 1 else 1)):
            run(f"mxfp8_M{m}", m, "rows/s", lambda inp=inp: omx.mxfp8_gemm(inp.x, inp.w, inp.s), threads, reps)
        del inp
    inp = workloads.moe_config("long_prompt")
    run("long_prompt", inp.T, "tokens/s", lambda: omoe.moe_layer(inp), logical, 1)
    rep = {"logical_cpus": logical, "physical_cores": physical, "rows": rows,
           "note": "fp64 NumPy oracle (test infrastructure, untuned); data generation excluded; BLAS threads "
                   "limited with threadpoolctl"}
    with open(path, "w") as fh:
        json.dump(rep, fh, indent=1)
    log(f"[cpu] wrote {path}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prompt", "long_prompt", "mxfp8_M1", "mxfp8_M512", "w8a8_M512",
                             "router_decode", "router_long_prompt", "block_decode", "block_long_prompt"])
    ap.add_argument("--rotations", type=int, default=0,
                    help="weight copies to rotate (0: enough for the touched weights to reach 1 GB)")
    ap.add_argument("--no-also", action="store_true", help="skip the prompt, long-prompt and MXFP8 measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also-steps", type=int, default=20)
    ap.add_argument("--cpu-protocol", default="",
                    help="only time the CPU oracle on every configuration and write this JSON file")
    args = ap.parse_args(argv)

    if args.cpu_protocol:
        cpu_protocol(args.cpu_protocol)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); multi-GPU sharding is a design "
              "note, not part of this build", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    import nvfp4_block_scaled_topk_amd as M
    import workloads
    M.lib()
    timer = Timer(torch)
    timer.calibrate_sleep()

    if args.workload.startswith("mxfp8_M"):
        # the MXFP8 projection alone (N=12288, K=4096): its own line, rows/s as the value
        m = int(args.workload[len("mxfp8_M"):])
        r = bench_mxfp8(m, args.steps, args.warmup, 20, timer)
        r["roofline"]["traffic"] = load_traffic(args.workload, MXFP8_FILES)
        print(json.dumps({
            "metric": METRIC, "value": r["rows_per_s"], "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": r["avg_us"] / 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"MXFP8 projection: M={m} bf16 rows, W 12288x4096 E4M3 in blocks of 32 with E8M0 scales"},
            "roofline": r["roofline"], "cpu_baseline": None}), flush=True)
        return

    if args.workload == "w8a8_M512":
        r = bench_w8a8(512, args.steps, args.warmup, 20, timer)
        print(json.dumps({
            "metric": METRIC, "value": r["rows_per_s"], "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": r["total_us"] / 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
            "config": {"workload": "W8A8 MXFP8 projection: M=512 bf16 rows quantized to MXFP8, W 12288x4096 E4M3 "
                                   "in blocks of 32 with E8M0 scales, block-scaled fp8 MFMA"},
            "roofline": r["roofline"], "cpu_baseline": None}), flush=True)
        return

    if args.workload.startswith("router_"):
        # the router projection alone: its own line, tokens/s as the value
        name = args.workload[len("router_"):]
        r = bench_router(name, args.steps, args.warmup, timer)
        print(json.dumps({
            "metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": r["avg_us"] / 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"router projection of the {name} MoE layer: T={r['T']} bf16 rows, "
                                   f"W_r bf16 {r['E']}x{r['d']}, fp32 logits"},
            "roofline": r["roofline"], "cpu_baseline": None}), flush=True)
        return

    if args.workload.startswith("block_"):
        # the whole MoE block (router, routing, routed and shared experts, combine): own line
        name = args.workload[len("block_"):]
        r = bench_block(name, args.steps, args.warmup, timer)
        decode_like = r["T"] <= 16
        roof = ({"bound": "hbm", "achieved": r["hbm_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                 "frac": r["hbm_gbps"] / HBM_PEAK_GBPS, "algorithmic_bytes": r["algorithmic_bytes"]}
                if decode_like else
                {"bound": "mfma", "achieved": r["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": r["tflops"] / BF16_PEAK_TFLOPS, "algorithmic_flop": r["algorithmic_flop"]})
        roof.update({"kernel": "whole block, one step", "avg_us": r["ms_per_step"] * 1e3, "traffic": None})
        print(json.dumps({
            "metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{name} MoE block: router projection, top-{r['k']} routing, {r['E']} routed NVFP4 "
                                   f"experts and one shared NVFP4 expert (T={r['T']}, d={r['d']}, f={r['f']}), "
                                   "gated shared add in the combine"},
            "roofline": roof, "cpu_baseline": None}), flush=True)
        return

    cid, T, d, f, E, k, zipf = workloads.MOE_CONFIGS[args.workload]
    main_res = bench_moe(args.workload, args.steps, args.warmup, args.rotations, timer)

    also = {}
    if not args.no_also and args.workload != "long_prompt":
        r = bench_moe("long_prompt", args.also_steps, 3, 0, timer)
        also["long_prompt"] = {
            "tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"], "touched_experts": r["touched_experts"],
            "roofline": {"bound": "mfma", "achieved": r["ffn_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": r["ffn_tflops"] / BF16_PEAK_TFLOPS, "traffic": load_traffic("long_prompt", PROMPT_FILES),
                         "kernel": PROMPT_KERNELS,
                         "algorithmic_flop": r["flops"], "avg_us": r["ffn_avg_us"]},
            "layer_tflops": r["layer_tflops"],
        }

    if not args.no_also and args.workload != "prompt":
        r = bench_moe("prompt", args.also_steps, 3, 0, timer)
        also["prompt"] = {
            "tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"], "touched_experts": r["touched_experts"],
            "ffn_avg_us": r["ffn_avg_us"], "ffn_hbm_gbps": r["ffn_hbm_gbps"],
            "ffn_hbm_frac": r["ffn_hbm_gbps"] / HBM_PEAK_GBPS, "ffn_tflops": r["ffn_tflops"],
            "ffn_mfma_frac": r["ffn_tflops"] / BF16_PEAK_TFLOPS,
            "ffn_traffic_bytes": load_traffic("prompt", PROMPT_FILES),
        }
    if not args.no_also:
        for m in (1, 512):
            r = bench_mxfp8(m, max(args.also_steps, 50), 5, 20, timer)
            r["roofline"]["traffic"] = load_traffic(f"mxfp8_M{m}", MXFP8_FILES)
            also[f"mxfp8_M{m}"] = r

    if not args.no_also:
        also["w8a8_M512"] = bench_w8a8(512, max(args.also_steps, 50), 5, 20, timer)
        also["mxfp8_columns"] = bench_mxfp8_columns(max(args.also_steps, 50), timer)
        also["ffn_pick"] = bench_ffn_pick()
        also["shards"] = bench_shards(max(args.also_steps, 50), timer)
        for name in ("decode", "long_prompt"):
            also[f"router_{name}"] = bench_router(name, max(args.also_steps, 50), 5, timer)
        also["block_decode"] = bench_block("decode", max(args.also_steps, 50), 5, timer)

    decode_like = main_res["T"] <= 16
    r = main_res
    if decode_like:
        files = DECODE_FILES
        roof = {"bound": "hbm", "achieved": r["launch_hbm_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": r["launch_hbm_gbps"] / HBM_PEAK_GBPS, "traffic": load_traffic(args.workload, files),
                "kernel": ("ffn_decode_kernel as moe_layer_nvfp4 runs it (routing, the expert FFN and the combine in "
                           "one launch: the only launch of a layer step)" if r["layer_in_one_launch"] else
                           "ffn_decode_kernel (moe_expert_ffn_nvfp4)"),
                "algorithmic_bytes": r["launch_bytes"], "avg_us": r["launch_us"],
                "separate_launches_us": r["separate_launches_us"],
                "layer_us": r["ms_per_step"] * 1e3, "layer_frac": r["layer_hbm_gbps"] / HBM_PEAK_GBPS,
                "ffn_alone_us": r["ffn_avg_us"], "ffn_alone_frac": r["ffn_hbm_gbps"] / HBM_PEAK_GBPS,
                "ceiling": {"kernel": "read_ranges_kernel (moe_read_ceiling: a plain coalesced read of the touched "
                                      "experts' codes and scales, same weight rotation, nothing else)",
                            "bytes": r["ceiling_bytes"], "avg_us": r["ceiling_us"], "gbps": r["ceiling_gbps"],
                            "frac_of_peak": r["ceiling_gbps"] / HBM_PEAK_GBPS,
                            "launch_frac_of_ceiling": r["launch_hbm_gbps"] / r["ceiling_gbps"]}}
    else:
        files = PROMPT_FILES
        roof = {"bound": "mfma", "achieved": r["ffn_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": r["ffn_tflops"] / BF16_PEAK_TFLOPS, "traffic": load_traffic(args.workload, files),
                "kernel": PROMPT_KERNELS, "algorithmic_flop": r["flops"], "avg_us": r["ffn_avg_us"],
                "layer_us": r["ms_per_step"] * 1e3,
                "ceiling": {"kernel": "read_ranges_kernel (moe_read_ceiling: the touched experts' bytes)",
                            "bytes": r["ceiling_bytes"], "avg_us": r["ceiling_us"], "gbps": r["ceiling_gbps"]}}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline()

    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} MoE layer: T={main_res['T']} tokens, d={main_res['d']}, "
                               f"f={main_res['f']}, E={main_res['E']} NVFP4 experts, top-{main_res['k']}"
                               + (", Zipf(1.1) routing skew" if zipf else ""),
                   "touched_experts": main_res["touched_experts"], "weight_copies_rotated": main_res["rotations"],
                   "layer_in_one_launch": main_res["layer_in_one_launch"],
                   "layer_hbm_gbps": main_res["layer_hbm_gbps"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_us": {"p10": r["step_us_p10"], "p50": r["step_us_p50"], "p90": r["step_us_p90"],
                    "note": "per-step durations from a second loop with an event between steps"},
    }
    if also:
        line["also"] = also
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
