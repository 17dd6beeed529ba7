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
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
# kernel sources whose hash a traffic record must match, per path
DECODE_FILES = ["ffn_decode.hip", "device.hpp"]
PROMPT_FILES = ["ffn_prompt.hip", "ffn_skinny.hip", "device.hpp"]
MXFP8_FILES = ["mxfp8.hip", "device.hpp"]
ROUTER_FILES = ["router.hip", "device.hpp"]
PROMPT_KERNELS = ("moe_expert_ffn_nvfp4 prompt path (ffn_prompt_kernel grouped GEMM gate/up + down; "
                  "ffn_skinny gate/up + down for experts with <= 16 rows)")


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
    # few tokens: routing runs inside the FFN launch (moe_route_expert_ffn_nvfp4) when the
    # shape allows it; otherwise route, then FFN
    fused = False
    if T <= 16:
        try:
            M.route_expert_ffn_nvfp4(logits, x, ex0, k, route_out=rbufs, out=y_rows, workspace=fws, check=False)
            fused = True
        except M.MoEError:
            fused = False

    def step(i, ev=None):
        ex = copies[i % rotations]
        if not fused:
            M.route_topk(logits, k, out=rbufs, workspace=rws)
        if ev is not None:
            ev[0].record()
        if fused:
            M.route_expert_ffn_nvfp4(logits, x, ex, k, route_out=rbufs, out=y_rows, workspace=fws, check=False)
        else:
            M.expert_ffn_nvfp4(x, ex, off, srows, k, out=y_rows, workspace=fws, check=False)
        if ev is not None:
            ev[1].record()
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

    # the FFN inside the layer, in a separate loop with an event pair around every FFN
    # call (the events add gaps to the layer, so this loop is not the timed region)
    n_ev = min(steps, 50)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    torch.cuda.synchronize()
    timer.queue_ahead(host_ms_per_step * n_ev * 1.5 + 20.0)
    for i in range(n_ev):
        step(i, evs[i])
    torch.cuda.synchronize()
    ffn_ms = [a.elapsed_time(b) for a, b in evs]
    ffn_in_layer_ms = sum(ffn_ms) / len(ffn_ms)

    # The expert FFN alone, back to back (same routing, rotating weight copies), between
    # one pair of events: its average duration per call, without per-call event overhead.
    n_ffn = max(steps, 20)
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    timer.queue_ahead(host_ms_per_step * n_ffn + 20.0)
    a_ev.record()
    for i in range(n_ffn):
        M.expert_ffn_nvfp4(x, copies[i % rotations], off, srows, k, out=y_rows, workspace=fws, check=False)
    b_ev.record()
    torch.cuda.synchronize()
    ffn_avg_ms = a_ev.elapsed_time(b_ev) / n_ffn

    # algorithmic work (only what the method must move / compute)
    eb = expert_bytes(d, f)
    ffn_bytes = U * eb + T * d * 2
    layer_bytes = U * eb + T * d * 2 + T * E * 4 + T * d * 2
    flops = 2.0 * T * k * 3 * d * f
    res = dict(
        name=name, T=T, d=d, f=f, E=E, k=k, touched_experts=U, rotations=rotations,
        ms_per_step=ms_per_step, tokens_per_s=T / (ms_per_step / 1e3),
        ffn_avg_us=ffn_avg_ms * 1e3, ffn_in_layer_us=ffn_in_layer_ms * 1e3, ffn_min_in_layer_us=min(ffn_ms) * 1e3,
        ffn_bytes=ffn_bytes, layer_bytes=layer_bytes, flops=flops,
        layer_hbm_gbps=layer_bytes / (ms_per_step / 1e3) / 1e9,
        ffn_hbm_gbps=ffn_bytes / (ffn_avg_ms / 1e3) / 1e9,
        ffn_tflops=flops / (ffn_avg_ms / 1e3) / 1e12,
        layer_tflops=flops / (ms_per_step / 1e3) / 1e12,
        host_ms_per_step=host_ms_per_step, route_in_ffn_launch=fused,
    )
    log(f"[bench] {name}: {json.dumps(res)}")
    del copies, ex0
    torch.cuda.empty_cache()
    return res


def bench_mxfp8(M, steps, warmup, rotations, timer, seed=0):
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
                           "kernel": "mxfp8_gemv_valu_kernel" if M <= 4 else "mxfp8_gemv_kernel",
                           "algorithmic_bytes": nbytes, "avg_us": res["avg_us"]}
    else:
        res["roofline"] = {"bound": "mfma", "achieved": res["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": res["tflops"] / BF16_PEAK_TFLOPS, "kernel": "mxfp8_gemm_kernel",
                           "algorithmic_flop": flops, "avg_us": res["avg_us"]}
    log(f"[bench] mxfp8 M={M}: {json.dumps(res)}")
    del ws, w0, s0
    torch.cuda.empty_cache()
    return res


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

    fused = False
    if T <= 16:
        try:
            M.route_expert_ffn_nvfp4(logits, x, ex0, k, route_out=rbufs, out=y_rows, workspace=fws, check=False)
            fused = True
        except M.MoEError:
            fused = False

    def step(i):
        ex, sx = copies[i % rotations]
        M.router_logits(x, w_r, out=logits)
        if fused:
            M.route_expert_ffn_nvfp4(logits, x, ex, k, route_out=rbufs, out=y_rows, workspace=fws, check=False)
        else:
            M.route_topk(logits, k, out=rbufs, workspace=rws)
            M.expert_ffn_nvfp4(x, ex, off, srows, k, out=y_rows, workspace=fws, check=False)
        M.shared_expert_nvfp4(x, sx, out=s_rows, workspace=sws)
        M.router_logits(x, w_sg, out=glog)
        M.combine(y_rows, rof, w, out=out, shared_rows=s_rows, shared_gate_logit=glog, residual=x)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(min(steps, 20)):
        step(i)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3 / min(steps, 20)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.queue_ahead(host_ms * steps * 1.5 + 20.0)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    nbytes = (U + 1) * eb + E * d * 2 + d * 2 + 2 * T * d * 2 + T * E * 4
    flops = 2.0 * T * (k + 1) * 3 * d * f + 2.0 * T * (E + 1) * d
    res = {"T": T, "d": d, "f": f, "E": E, "k": k, "touched_experts": U, "weight_copies_rotated": rotations,
           "route_in_ffn_launch": fused,
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


def cpu_baseline(budget_s=12.0):
    """The oracle (test infrastructure, untuned) on the host cores: whole decode
    layers (route, dequantize, FFN, combine) on the same seeded input, repeated
    until about `budget_s` of CPU time."""
    import workloads
    from oracle import moe as omoe

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    inp = workloads.moe_config("decode")
    reps = 0
    t0 = time.perf_counter()
    while True:
        omoe.moe_layer(inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": reps * inp.T / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} whole decode layers (T={inp.T}, d={inp.d}, f={inp.f}, E={inp.E}, k={inp.k}) "
                      f"in {el:.1f} s; fp64 NumPy, BLAS matmuls on {threads} threads, the rest single-threaded"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prompt", "long_prompt", "mxfp8_M1", "mxfp8_M512",
                             "router_decode", "router_long_prompt", "block_decode", "block_long_prompt"])
    ap.add_argument("--rotations", type=int, default=0,
                    help="weight copies to rotate (0: enough for the touched weights to reach 1 GB)")
    ap.add_argument("--no-also", action="store_true", help="skip the prompt, long-prompt and MXFP8 measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also-steps", type=int, default=20)
    args = ap.parse_args(argv)

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
        for name in ("decode", "long_prompt"):
            also[f"router_{name}"] = bench_router(name, max(args.also_steps, 50), 5, timer)
        also["block_decode"] = bench_block("decode", max(args.also_steps, 50), 5, timer)

    decode_like = main_res["T"] <= 16
    if decode_like:
        files = DECODE_FILES
        roof = {"bound": "hbm", "achieved": main_res["ffn_hbm_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": main_res["ffn_hbm_gbps"] / HBM_PEAK_GBPS, "traffic": load_traffic(args.workload, files),
                "kernel": "moe_expert_ffn_nvfp4 decode (ffn_decode_kernel: gate/up/SwiGLU and down in one launch)",
                "algorithmic_bytes": main_res["ffn_bytes"], "avg_us": main_res["ffn_avg_us"],
                "avg_us_in_layer": main_res["ffn_in_layer_us"]}
    else:
        files = PROMPT_FILES
        roof = {"bound": "mfma", "achieved": main_res["ffn_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": main_res["ffn_tflops"] / BF16_PEAK_TFLOPS, "traffic": load_traffic(args.workload, files),
                "kernel": PROMPT_KERNELS,
                "algorithmic_flop": main_res["flops"], "avg_us": main_res["ffn_avg_us"],
                "avg_us_in_layer": main_res["ffn_in_layer_us"]}

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
                   "route_in_ffn_launch": main_res["route_in_ffn_launch"],
                   "layer_hbm_gbps": main_res["layer_hbm_gbps"]},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if also:
        line["also"] = also
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
