"""Routed NVFP4 mixture-of-experts FFN and MXFP8 projection for AMD Instinct MI355X.

A thin Python binding over the C ABI of libmoe_nvfp4.so (include/moe_nvfp4.h):
argument marshalling only. Every step of the layer runs in the library's HIP
kernels; torch supplies device memory and the current stream. There is no CPU
fallback: without the built library every call raises.

    logits = router_logits(x, w_r)
    ids, w, offsets, sorted_rows, row_of = route_topk(logits, k)
    y_rows = expert_ffn_nvfp4(x, experts, offsets, sorted_rows, k)
    out = combine(y_rows, row_of, w)
    y = mxfp8_gemm(x, w_e4m3, s_e8m0)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_nvfp4.so")

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_E_NULL", 2: "MOE_E_SHAPE", 3: "MOE_E_ALIGN",
                4: "MOE_E_WORKSPACE", 5: "MOE_E_LAUNCH", 6: "MOE_E_POLICY", 7: "MOE_E_WAIT_EXPIRED"}
# routing normalization policies (MOE_ROUTE_* in the header)
ROUTE_SOFTMAX_RENORM, ROUTE_SOFTMAX, ROUTE_SIGMOID_RENORM, ROUTE_SIGMOID = 0, 1, 2, 3

EXPORTED_SYMBOLS = (
    "moe_route_topk_workspace", "moe_route_topk", "moe_route_topk_policy", "moe_expert_ffn_nvfp4_workspace",
    "moe_expert_ffn_nvfp4", "moe_route_expert_ffn_nvfp4", "moe_combine", "moe_combine_shared", "mxfp8_gemm", "moe_router_logits", "moe_status_string",
    "moe_last_error", "moe_async_status", "moe_set_wait_limits", "moe_get_wait_limits",
    "moe_expert_ffn_nvfp4_scratch", "moe_combine_residual", "moe_read_ceiling", "mxfp8_quantize", "mxfp8_gemm_mx",
    "mxfp8_autotune", "mxfp8_force_kernel", "moe_layer_nvfp4_workspace", "moe_layer_nvfp4", "moe_ffn_autotune",
    "moe_ffn_force_path",
)


class MoEError(RuntimeError):
    """A non-zero status from the library, named."""

    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{where}: {name}" + (f" ({detail})" if detail else ""))


class _Experts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m nvfp4_block_scaled_topk_amd.build` (there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.moe_route_topk_workspace.argtypes = [i32, i32, i32]
    L.moe_route_topk_workspace.restype = sz
    L.moe_route_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_topk.restype = i32
    L.moe_route_topk_policy.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_topk_policy.restype = i32
    L.moe_expert_ffn_nvfp4_workspace.argtypes = [i32, i32, i32, i32, i32]
    L.moe_expert_ffn_nvfp4_workspace.restype = sz
    L.moe_expert_ffn_nvfp4.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(_Experts), vp, vp, vp,
                                       vp, sz, vp]
    L.moe_expert_ffn_nvfp4.restype = i32
    L.moe_expert_ffn_nvfp4_scratch.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(_Experts), vp, vp, vp,
                                               vp]
    L.moe_expert_ffn_nvfp4_scratch.restype = i32
    L.moe_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
    L.moe_combine.restype = i32
    L.moe_route_expert_ffn_nvfp4.argtypes = [vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(_Experts),
                                             vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_expert_ffn_nvfp4.restype = i32
    L.moe_combine_residual.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.moe_combine_residual.restype = i32
    L.moe_combine_shared.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    L.moe_combine_shared.restype = i32
    L.mxfp8_gemm.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    L.mxfp8_gemm.restype = i32
    L.moe_router_logits.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    L.moe_router_logits.restype = i32
    L.moe_async_status.argtypes = [vp]
    L.moe_async_status.restype = i32
    L.moe_set_wait_limits.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    L.moe_set_wait_limits.restype = None
    L.moe_get_wait_limits.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    L.moe_get_wait_limits.restype = None
    L.mxfp8_autotune.argtypes = [vp, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp]
    L.mxfp8_autotune.restype = i32
    L.mxfp8_force_kernel.argtypes = [i32]
    L.mxfp8_force_kernel.restype = i32
    L.mxfp8_quantize.argtypes = [vp, i32, i32, vp, vp, vp]
    L.mxfp8_quantize.restype = i32
    L.mxfp8_gemm_mx.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
    L.mxfp8_gemm_mx.restype = i32
    L.moe_read_ceiling.argtypes = [vp, i32, ctypes.c_uint64, vp, i32, vp]
    L.moe_read_ceiling.restype = i32
    L.moe_layer_nvfp4_workspace.argtypes = [i32, i32, i32, i32, i32, i32]
    L.moe_layer_nvfp4_workspace.restype = sz
    L.moe_layer_nvfp4.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, ctypes.POINTER(_Experts),
                                  ctypes.POINTER(_Experts), vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_layer_nvfp4.restype = i32
    L.moe_ffn_autotune.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(_Experts), vp, vp, vp, vp, sz, i32,
                                   vp, vp, vp]
    L.moe_ffn_autotune.restype = i32
    L.moe_ffn_force_path.argtypes = [i32]
    L.moe_ffn_force_path.restype = i32
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        detail = lib().moe_last_error().decode() if status == 5 else ""
        raise MoEError(status, where, detail)


def async_status(device=None) -> int:
    """Waits for torch's current stream and returns the library's asynchronous status
    (0, or 7 = MOE_E_WAIT_EXPIRED: a few-token launch gave up a wait; the affected rows
    are NaN), clearing it."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        st = lib().moe_async_status(torch.cuda.current_stream(dev).cuda_stream)
    if st not in (0, 7):
        _check(st, "moe_async_status")
    return st


def wait_limits() -> tuple:
    """(steal_after, give_up): the polls of the few-token launch's waits."""
    a, b = ctypes.c_uint32(), ctypes.c_uint32()
    lib().moe_get_wait_limits(ctypes.byref(a), ctypes.byref(b))
    return int(a.value), int(b.value)


def set_wait_limits(steal_after: int, give_up: int) -> tuple:
    """Sets the polls of the few-token launch's waits (see moe_set_wait_limits); returns
    the previous (steal_after, give_up)."""
    prev = wait_limits()
    lib().moe_set_wait_limits(int(steal_after), int(give_up))
    return prev


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


@dataclass
class NVFP4Experts:
    """E routed experts as stored: uint8 codes / E4M3 scales, fp32 tensor scales.

    gate_q, up_q: [E, f, d/2]; gate_s, up_s: [E, f, d/16]; down_q: [E, d, f/2];
    down_s: [E, d, f/16]; gate_ts, up_ts, down_ts: [E] float32.
    """

    gate_q: torch.Tensor
    gate_s: torch.Tensor
    gate_ts: torch.Tensor
    up_q: torch.Tensor
    up_s: torch.Tensor
    up_ts: torch.Tensor
    down_q: torch.Tensor
    down_s: torch.Tensor
    down_ts: torch.Tensor

    @property
    def E(self):
        return self.gate_q.shape[0]

    @property
    def f(self):
        return self.gate_q.shape[1]

    @property
    def d(self):
        return self.gate_q.shape[2] * 2

    def check(self):
        E, f, d = self.E, self.f, self.d
        _dev(self.gate_q, torch.uint8, "gate_q", (E, f, d // 2))
        _dev(self.up_q, torch.uint8, "up_q", (E, f, d // 2))
        _dev(self.gate_s, torch.uint8, "gate_s", (E, f, d // 16))
        _dev(self.up_s, torch.uint8, "up_s", (E, f, d // 16))
        _dev(self.down_q, torch.uint8, "down_q", (E, d, f // 2))
        _dev(self.down_s, torch.uint8, "down_s", (E, d, f // 16))
        for n in ("gate_ts", "up_ts", "down_ts"):
            _dev(getattr(self, n), torch.float32, n, (E,))

    def c_struct(self) -> _Experts:
        return _Experts(*[getattr(self, n).data_ptr() for n in
                          ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")])

    @classmethod
    def from_numpy(cls, inp, device="cuda"):
        """Upload the expert arrays of a workloads.MoEInputs-like object."""
        def t(a):
            return torch.from_numpy(a).to(device)
        return cls(*[t(getattr(inp, n)) for n in
                     ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts")])


def read_ceiling(ranges: torch.Tensor, total_bytes: int, sink: torch.Tensor):
    """A plain streaming read of byte ranges (a measurement helper): `ranges` int64 device
    tensor [n, 2] of (address, bytes), `sink` int32 device tensor (one word a workgroup)."""
    n = ranges.shape[0]
    st = lib().moe_read_ceiling(_dev(ranges, torch.int64, "ranges", (n, 2)), n, int(total_bytes),
                                _dev(sink, torch.int32, "sink"), sink.numel(), _stream(ranges))
    _check(st, "moe_read_ceiling")


def route_topk_workspace(T: int, E: int, k: int) -> int:
    return int(lib().moe_route_topk_workspace(T, E, k))


def route_topk(logits: torch.Tensor, k: int, out=None, workspace=None, policy: int = ROUTE_SOFTMAX_RENORM,
               bias: torch.Tensor | None = None):
    """Top-k routing and row lists. Returns (ids int32 [T,k], w fp32 [T,k],
    offsets int32 [E+1], sorted_rows int32 [T*k], row_of int32 [T*k]). `policy` is a
    ROUTE_* normalization policy; `bias` (fp32 [E]) a correction bias on the choice."""
    T, E = logits.shape
    lp = _dev(logits, torch.float32, "logits")
    dev = logits.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((E + 1,), dtype=torch.int32, device=dev), torch.empty((T * k,), dtype=torch.int32, device=dev),
               torch.empty((T * k,), dtype=torch.int32, device=dev))
    ids, w, off, srows, rof = out
    need = route_topk_workspace(T, E, k)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    wsp = workspace.data_ptr() if workspace is not None else None
    wsb = workspace.numel() if workspace is not None else 0
    outs = (_dev(ids, torch.int32, "ids", (T, k)), _dev(w, torch.float32, "w", (T, k)),
            _dev(off, torch.int32, "offsets", (E + 1,)), _dev(srows, torch.int32, "sorted_rows", (T * k,)),
            _dev(rof, torch.int32, "row_of", (T * k,)))
    if policy == ROUTE_SOFTMAX_RENORM and bias is None:
        st = lib().moe_route_topk(lp, T, E, k, *outs, wsp, wsb, _stream(logits))
        _check(st, "moe_route_topk")
    else:
        bp = _dev(bias, torch.float32, "bias", (E,)) if bias is not None else None
        st = lib().moe_route_topk_policy(lp, T, E, k, int(policy), bp, *outs, wsp, wsb, _stream(logits))
        _check(st, "moe_route_topk_policy")
    return ids, w, off, srows, rof


def expert_ffn_workspace(T: int, d: int, f: int, E: int, k: int) -> int:
    return int(lib().moe_expert_ffn_nvfp4_workspace(T, d, f, E, k))


def expert_ffn_nvfp4(x: torch.Tensor, experts: NVFP4Experts, offsets: torch.Tensor, sorted_rows: torch.Tensor,
                     k: int, out=None, workspace=None, check: bool = True):
    """Expert FFN of every routed row; x is bf16 [T, d] (torch.bfloat16 or its
    uint16/int16 bits). Returns y_rows fp32 [T*k, d] in row-list order."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    T, d = x.shape
    E, f = experts.E, experts.f
    if experts.d != d:
        raise ValueError(f"x has d={d}, experts have d={experts.d}")
    if check:
        experts.check()
    dev = x.device
    if out is None:
        out = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    need = expert_ffn_workspace(T, d, f, E, k)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    ex = experts.c_struct()
    st = lib().moe_expert_ffn_nvfp4(_dev(x, torch.bfloat16, "x"), T, d, f, E, k, ctypes.byref(ex),
                                    _dev(offsets, torch.int32, "offsets", (E + 1,)),
                                    _dev(sorted_rows, torch.int32, "sorted_rows", (T * k,)),
                                    _dev(out, torch.float32, "y_rows", (T * k, d)), workspace.data_ptr(),
                                    workspace.numel(), _stream(x))
    _check(st, "moe_expert_ffn_nvfp4")
    return out


# bytes of the static scratch behind expert_ffn_nvfp4_scratch (MOE_SCRATCH_BYTES)
SCRATCH_BYTES = 32 << 20


def expert_ffn_nvfp4_scratch(x: torch.Tensor, experts: NVFP4Experts, offsets: torch.Tensor,
                             sorted_rows: torch.Tensor, k: int, out: torch.Tensor, check: bool = True):
    """expert_ffn_nvfp4 through moe_expert_ffn_nvfp4_scratch: no workspace and no allocation
    (the caller passes `out`, y_rows fp32 [T*k, d]); H lives in the library's static
    scratch of SCRATCH_BYTES a device. Calls that overlap on one device race."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    T, d = x.shape
    E, f = experts.E, experts.f
    if experts.d != d:
        raise ValueError(f"x has d={d}, experts have d={experts.d}")
    if check:
        experts.check()
    ex = experts.c_struct()
    st = lib().moe_expert_ffn_nvfp4_scratch(_dev(x, torch.bfloat16, "x"), T, d, f, E, k, ctypes.byref(ex),
                                            _dev(offsets, torch.int32, "offsets", (E + 1,)),
                                            _dev(sorted_rows, torch.int32, "sorted_rows", (T * k,)),
                                            _dev(out, torch.float32, "y_rows", (T * k, d)), _stream(x))
    if st == 4:
        raise MoEError(st, "moe_expert_ffn_nvfp4_scratch", lib().moe_last_error().decode())
    _check(st, "moe_expert_ffn_nvfp4_scratch")
    return out


def combine(y_rows: torch.Tensor, row_of: torch.Tensor, w: torch.Tensor, out=None,
            shared_rows: torch.Tensor | None = None, shared_gate_logit: torch.Tensor | None = None,
            residual: torch.Tensor | None = None):
    """out bf16 [T, d] = bf16_rne(sum_j w[t, j] * y_rows[row_of[t*k + j]] (+ g_t * shared_rows[t],
    g_t = sigmoid(shared_gate_logit[t]) or 1) (+ residual[t], bf16 [T, d]))."""
    T, k = w.shape
    d = y_rows.shape[1]
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=y_rows.device)
    if residual is not None:
        if residual.dtype in (torch.uint16, torch.int16):
            residual = residual.view(torch.bfloat16)
        sp = _dev(shared_rows, torch.float32, "shared_rows", (T, d)) if shared_rows is not None else None
        gp = None
        if shared_gate_logit is not None:
            gp = _dev(shared_gate_logit.reshape(T), torch.float32, "shared_gate_logit", (T,))
        st = lib().moe_combine_residual(_dev(y_rows, torch.float32, "y_rows", (T * k, d)),
                                        _dev(row_of, torch.int32, "row_of", (T * k,)),
                                        _dev(w, torch.float32, "w", (T, k)), T, k, d, sp, gp,
                                        _dev(residual, torch.bfloat16, "residual", (T, d)),
                                        _dev(out, torch.bfloat16, "out", (T, d)), _stream(y_rows))
        _check(st, "moe_combine_residual")
        return out
    if shared_rows is not None:
        gp = None
        if shared_gate_logit is not None:
            gp = _dev(shared_gate_logit.reshape(T), torch.float32, "shared_gate_logit", (T,))
        st = lib().moe_combine_shared(_dev(y_rows, torch.float32, "y_rows", (T * k, d)),
                                      _dev(row_of, torch.int32, "row_of", (T * k,)), _dev(w, torch.float32, "w", (T, k)),
                                      T, k, d, _dev(shared_rows, torch.float32, "shared_rows", (T, d)), gp,
                                      _dev(out, torch.bfloat16, "out", (T, d)), _stream(y_rows))
        _check(st, "moe_combine_shared")
        return out
    st = lib().moe_combine(_dev(y_rows, torch.float32, "y_rows", (T * k, d)), _dev(row_of, torch.int32, "row_of", (T * k,)),
                           _dev(w, torch.float32, "w", (T, k)), T, k, d, _dev(out, torch.bfloat16, "out", (T, d)),
                           _stream(y_rows))
    _check(st, "moe_combine")
    return out


def moe_layer(x: torch.Tensor, logits: torch.Tensor, experts: NVFP4Experts, k: int):
    """Route, expert FFN, combine: the whole routed MoE FFN. Returns out bf16 [T, d]. For a
    few tokens (the shapes moe_layer_nvfp4 takes) this is one launch, with the same bits as
    the three calls it replaces."""
    T, d = x.shape
    if layer_workspace(T, d, experts.f, experts.E, k) > 0:
        return layer_nvfp4(logits, x, experts, k)
    ids, w, off, srows, rof = route_topk(logits, k)
    y_rows = expert_ffn_nvfp4(x, experts, off, srows, k)
    return combine(y_rows, rof, w)


def mxfp8_gemm(x: torch.Tensor, w: torch.Tensor, s: torch.Tensor, out=None):
    """y bf16 [M, N] = x . W^T with W = E4M3(w) * 2^(s - 127) per 32-element block."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    st = lib().mxfp8_gemm(_dev(x, torch.bfloat16, "x"), M, N, K, _dev(w, torch.uint8, "w", (N, K)),
                          _dev(s, torch.uint8, "s", (N, K // 32)), _dev(out, torch.bfloat16, "y", (M, N)),
                          _stream(x))
    _check(st, "mxfp8_gemm")
    return out


MXFP8_KERNELS = ("vector-ALU gemv", "MFMA gemv", "tiled GEMM")


def mxfp8_autotune(x: torch.Tensor, w: torch.Tensor, s: torch.Tensor, reps: int = 20):
    """Times the few-row MXFP8 kernels for M = 1 .. x.shape[0] (<= 16) on these operands
    and records the fastest per (device, M, N, K). Returns (picks [M_max] kernel ids,
    microseconds [M_max][3], NaN where a kernel was not timed)."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    M_max, K = x.shape
    N = w.shape[0]
    y = torch.empty((M_max, N), dtype=torch.bfloat16, device=x.device)
    picks = (ctypes.c_int * M_max)()
    us = (ctypes.c_float * (3 * M_max))(*([float("nan")] * (3 * M_max)))
    st = lib().mxfp8_autotune(_dev(x, torch.bfloat16, "x"), M_max, N, K, _dev(w, torch.uint8, "w", (N, K)),
                              _dev(s, torch.uint8, "s", (N, K // 32)), _dev(y, torch.bfloat16, "y", (M_max, N)),
                              int(reps), picks, us, _stream(x))
    _check(st, "mxfp8_autotune")
    return list(picks), [list(us[3 * i:3 * i + 3]) for i in range(M_max)]


def mxfp8_force_kernel(kernel: int):
    """Test hook: run the given few-row MXFP8 kernel id for every M <= 16 (-1: the records)."""
    _check(lib().mxfp8_force_kernel(int(kernel)), "mxfp8_force_kernel")


def mxfp8_quantize(x: torch.Tensor, out=None):
    """bf16 activations [M, K] -> (xq uint8 [M, K] E4M3 codes, xs uint8 [M, K/32] E8M0 scales),
    the OCP MX conversion (W8A8 variant)."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    M, K = x.shape
    if out is None:
        out = (torch.empty((M, K), dtype=torch.uint8, device=x.device),
               torch.empty((M, K // 32), dtype=torch.uint8, device=x.device))
    xq, xs = out
    st = lib().mxfp8_quantize(_dev(x, torch.bfloat16, "x"), M, K, _dev(xq, torch.uint8, "xq", (M, K)),
                              _dev(xs, torch.uint8, "xs", (M, K // 32)), _stream(x))
    _check(st, "mxfp8_quantize")
    return xq, xs


def mxfp8_gemm_mx(xq: torch.Tensor, xs: torch.Tensor, w: torch.Tensor, s: torch.Tensor, out=None):
    """y bf16 [M, N] = X . W^T with MXFP8 activations (xq, xs) and MXFP8 weights (w, s)."""
    M, K = xq.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    st = lib().mxfp8_gemm_mx(_dev(xq, torch.uint8, "xq", (M, K)), _dev(xs, torch.uint8, "xs", (M, K // 32)), M, N, K,
                             _dev(w, torch.uint8, "w", (N, K)), _dev(s, torch.uint8, "s", (N, K // 32)),
                             _dev(out, torch.bfloat16, "y", (M, N)), _stream(xq))
    _check(st, "mxfp8_gemm_mx")
    return out


def router_logits(x: torch.Tensor, w_r: torch.Tensor, out=None):
    """logits fp32 [T, E] = x . W_r^T, x bf16 [T, d], W_r bf16 [E, d] (fp32 accumulation)."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    if w_r.dtype in (torch.uint16, torch.int16):
        w_r = w_r.view(torch.bfloat16)
    T, d = x.shape
    E = w_r.shape[0]
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    st = lib().moe_router_logits(_dev(x, torch.bfloat16, "x"), _dev(w_r, torch.bfloat16, "w_r", (E, d)), T, d, E,
                                 _dev(out, torch.float32, "logits", (T, E)), _stream(x))
    _check(st, "moe_router_logits")
    return out


_shared_lists = {}


def shared_expert_nvfp4(x: torch.Tensor, shared: NVFP4Experts, out=None, workspace=None):
    """The shared expert's rows S fp32 [T, d]: moe_expert_ffn_nvfp4 with one expert that every
    token routes to (offsets {0, T}, row p = token p). The two index lists are constants of
    T, built once per (T, device)."""
    if shared.E != 1:
        raise ValueError("a shared expert is one expert (leading axis 1)")
    T = x.shape[0]
    key = (T, x.device)
    if key not in _shared_lists:
        _shared_lists[key] = (torch.tensor([0, T], dtype=torch.int32, device=x.device),
                              torch.arange(T, dtype=torch.int32, device=x.device))
    off, rows = _shared_lists[key]
    return expert_ffn_nvfp4(x, shared, off, rows, 1, out=out, workspace=workspace)


def route_expert_ffn_nvfp4(logits: torch.Tensor, x: torch.Tensor, experts: NVFP4Experts, k: int,
                           route_out=None, out=None, workspace=None, check: bool = True):
    """Routing and the expert FFN in one launch (few tokens: T <= 16, E <= 256, k <= 16).
    Returns ((ids, w, offsets, sorted_rows, row_of), y_rows) as route_topk and
    expert_ffn_nvfp4 would."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    T, E = logits.shape
    d = x.shape[1]
    f = experts.f
    dev = x.device
    if check:
        experts.check()
    if route_out is None:
        route_out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
                     torch.empty((E + 1,), dtype=torch.int32, device=dev), torch.empty((T * k,), dtype=torch.int32, device=dev),
                     torch.empty((T * k,), dtype=torch.int32, device=dev))
    ids, w, off, srows, rof = route_out
    if out is None:
        out = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty((max(expert_ffn_workspace(T, d, f, E, k), 1),), dtype=torch.uint8, device=dev)
    cs = experts.c_struct()
    st = lib().moe_route_expert_ffn_nvfp4(
        _dev(logits, torch.float32, "logits", (T, E)), _dev(x, torch.bfloat16, "x", (T, d)), T, d, f, E, k,
        ctypes.byref(cs), _dev(ids, torch.int32, "ids", (T, k)), _dev(w, torch.float32, "w", (T, k)),
        _dev(off, torch.int32, "offsets", (E + 1,)), _dev(srows, torch.int32, "sorted_rows", (T * k,)),
        _dev(rof, torch.int32, "row_of", (T * k,)), _dev(out, torch.float32, "y_rows", (T * k, d)),
        workspace.data_ptr(), workspace.numel(), _stream(x))
    _check(st, "moe_route_expert_ffn_nvfp4")
    return route_out, out


FFN_PATHS = ("decode launch", "streaming kernels")


def ffn_autotune(x: torch.Tensor, experts: NVFP4Experts, expert_offsets: torch.Tensor, sorted_rows: torch.Tensor,
                 k: int, reps: int = 20):
    """Times the two few-token paths of expert_ffn_nvfp4 (T <= 16) on these operands and
    routing and records the faster for this card and shape (moe_ffn_autotune). Returns
    (pick, us): the path recorded and the microseconds a call of each path (NaN where a
    path was not timed)."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    T, d = x.shape
    E, f = experts.E, experts.f
    y = torch.empty((T * k, d), dtype=torch.float32, device=x.device)
    ws = torch.empty((max(expert_ffn_workspace(T, d, f, E, k), 1),), dtype=torch.uint8, device=x.device)
    pick = ctypes.c_int(-1)
    us = (ctypes.c_float * 2)(float("nan"), float("nan"))
    cs = experts.c_struct()
    st = lib().moe_ffn_autotune(
        _dev(x, torch.bfloat16, "x", (T, d)), T, d, f, E, k, ctypes.byref(cs),
        _dev(expert_offsets, torch.int32, "expert_offsets", (E + 1,)),
        _dev(sorted_rows, torch.int32, "sorted_rows", (T * k,)), y.data_ptr(), ws.data_ptr(), ws.numel(), reps,
        ctypes.byref(pick), us, _stream(x))
    _check(st, "moe_ffn_autotune")
    return pick.value, [us[0], us[1]]


def ffn_force_path(path: int):
    """Test hook: force the few-token path of expert_ffn_nvfp4 (0 decode launch, 1 streaming
    kernels), or follow the records again (-1)."""
    _check(lib().moe_ffn_force_path(path), "moe_ffn_force_path")


def layer_workspace(T: int, d: int, f: int, E: int, k: int, shared: bool = False) -> int:
    """Workspace bytes of moe_layer_nvfp4 (0: the shape is not a few-token shape)."""
    return int(lib().moe_layer_nvfp4_workspace(T, d, f, E, k, 1 if shared else 0))


def layer_nvfp4(logits: torch.Tensor, x: torch.Tensor, experts: NVFP4Experts, k: int, shared: NVFP4Experts = None,
                shared_gate_logit: torch.Tensor = None, residual: torch.Tensor = None, route_out=None, out=None,
                workspace=None, check: bool = True):
    """The whole routed layer for few tokens in one launch (moe_layer_nvfp4): routing,
    the routed experts' FFN, an optional shared expert, and the combine with its gated
    shared add and an optional residual: out = bf16_rne(sum_j w_j O_j (+ g S) (+ residual)),
    the same bits as route_topk, expert_ffn_nvfp4 (and shared_expert_nvfp4) and combine.
    logits float32 [T, L] with L >= E (columns past E are not read: the shared gate's
    logit may sit in column E); shared_gate_logit float32 [T] or a [T, 1] column view of a
    row-major float32 tensor (g = 1 when absent); residual bf16 [T, d]. route_out, when
    given, receives (ids, w, offsets, sorted_rows, row_of). A workspace passed in must have
    been zero-filled before its first use (torch.zeros); calls leave it reusable. Returns
    out bf16 [T, d]."""
    if x.dtype in (torch.uint16, torch.int16):
        x = x.view(torch.bfloat16)
    T, d = x.shape
    E, f = experts.E, experts.f
    dev = x.device
    if logits.dim() != 2 or logits.shape[0] != T or logits.shape[1] < E or logits.dtype != torch.float32 or \
            not logits.is_cuda or not logits.is_contiguous():
        raise ValueError(f"logits must be a contiguous float32 CUDA tensor [T={T}, >= E={E}]")
    if check:
        experts.check()
        if shared is not None:
            shared.check()
    if shared is not None and (shared.E != 1 or shared.f != f or shared.d != d):
        raise ValueError("the shared expert is one expert of the routed experts' d and f")
    gptr, gld = None, 1
    if shared_gate_logit is not None:
        g = shared_gate_logit
        if not g.is_cuda or g.dtype != torch.float32 or g.shape[0] != T or g.numel() != T or \
                (g.dim() == 2 and g.shape[1] != 1) or g.dim() > 2:
            raise ValueError(f"shared_gate_logit must be float32 [T={T}] or [T, 1] on the device")
        gptr, gld = g.data_ptr(), (g.stride(0) if T > 1 else 1)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    need = layer_workspace(T, d, f, E, k, shared is not None)
    if workspace is None:  # zero-filled before its first use (the arrival counters)
        workspace = torch.zeros((max(need, 1),), dtype=torch.uint8, device=dev)
    rp = [None] * 5
    if route_out is not None:
        ids, w, off, srows, rof = route_out
        rp = [_dev(ids, torch.int32, "ids", (T, k)), _dev(w, torch.float32, "w", (T, k)),
              _dev(off, torch.int32, "offsets", (E + 1,)), _dev(srows, torch.int32, "sorted_rows", (T * k,)),
              _dev(rof, torch.int32, "row_of", (T * k,))]
    cs = experts.c_struct()
    ss = shared.c_struct() if shared is not None else None
    rptr = _dev(residual.view(torch.bfloat16) if residual is not None and residual.dtype != torch.bfloat16
                else residual, torch.bfloat16, "residual", (T, d)) if residual is not None else None
    st = lib().moe_layer_nvfp4(
        logits.data_ptr(), logits.shape[1], _dev(x, torch.bfloat16, "x", (T, d)), T, d, f, E, k, ctypes.byref(cs),
        ctypes.byref(ss) if ss is not None else None, gptr, gld, rptr, *rp,
        _dev(out, torch.bfloat16, "out", (T, d)), workspace.data_ptr(), workspace.numel(), _stream(x))
    _check(st, "moe_layer_nvfp4")
    return out

