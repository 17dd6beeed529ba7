"""The C-ABI library loads, exports every function include/moe_nvfp4.h declares,
and refuses bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_topk_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH), reason="library not built")

OK, NULL, SHAPE, ALIGN, WS = 0, 1, 2, 3, 4
A = 0x10000  # a 16-byte-aligned fake address: only ever passed to calls that must refuse


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) == set(M.EXPORTED_SYMBOLS), names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(M.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings():
    L = M.lib()
    for code, name in M.STATUS_NAMES.items():
        assert L.moe_status_string(code).decode() == name
    assert L.moe_status_string(99).decode() == "MOE_E_UNKNOWN"


def test_route_refusals():
    L = M.lib()
    f = L.moe_route_topk
    good = dict(logits=A, T=4, E=8, k=2, ids=A, w=A, off=A, sr=A, ro=A, ws=None, wsb=0, st=None)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["logits"], a["T"], a["E"], a["k"], a["ids"], a["w"], a["off"], a["sr"], a["ro"], a["ws"], a["wsb"], a["st"])
    assert call(logits=None) == NULL
    assert call(ro=None) == NULL
    assert call(T=0) == SHAPE
    assert call(E=0) == SHAPE
    assert call(E=1025, k=2) == SHAPE
    assert call(k=0) == SHAPE
    assert call(k=9) == SHAPE          # k > E
    assert call(E=64, k=33) == SHAPE   # k > 32
    assert call(logits=A + 4) == ALIGN
    assert call(off=A + 8) == ALIGN
    # more than one 16-token block needs a workspace
    need = L.moe_route_topk_workspace(17, 8, 2)
    assert need > 0
    assert L.moe_route_topk_workspace(16, 8, 2) == 0
    assert call(T=17) == WS
    assert call(T=17, ws=A, wsb=need - 1) == WS
    assert call(T=17, ws=A + 4, wsb=need) == ALIGN
    assert L.moe_route_topk_workspace(0, 8, 2) == 0


def test_ffn_refusals():
    L = M.lib()
    ex = M._Experts(*([A] * 9))
    T, d, f, E, k = 4, 256, 128, 8, 2
    need = L.moe_expert_ffn_nvfp4_workspace(T, d, f, E, k)
    assert need >= T * k * f * 2 and need % 256 == 0

    def call(x=A, T=T, d=d, f=f, E=E, k=k, ex=ex, off=A, sr=A, y=A, ws=A, wsb=need):
        return L.moe_expert_ffn_nvfp4(x, T, d, f, E, k, ctypes.byref(ex) if ex is not None else None,
                                      off, sr, y, ws, wsb, None)
    assert call(x=None) == NULL
    assert call(ex=None) == NULL
    bad = M._Experts(*([A] * 8 + [0]))
    assert call(ex=bad) == NULL
    assert call(d=48) == SHAPE
    assert call(f=16) == SHAPE
    assert call(E=1025) == SHAPE
    assert call(k=9) == SHAPE
    assert call(T=0) == SHAPE
    mis = M._Experts(*([A] * 4 + [A + 2] + [A] * 4))
    assert call(ex=mis) == ALIGN
    assert call(y=A + 4) == ALIGN
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=A + 8) == ALIGN


def test_combine_and_mxfp8_refusals():
    L = M.lib()
    assert L.moe_combine(None, A, A, 4, 2, 64, A, None) == NULL
    assert L.moe_combine(A, A, A, 4, 33, 64, A, None) == SHAPE
    assert L.moe_combine(A, A, A, 4, 2, 48, A, None) == SHAPE
    assert L.moe_combine(A, A, A + 4, 4, 2, 64, A, None) == ALIGN
    assert L.mxfp8_gemm(A, 1, 16, 64, None, A, A, None) == NULL
    assert L.mxfp8_gemm(A, 1, 16, 48, A, A, A, None) == SHAPE
    assert L.mxfp8_gemm(A, 0, 16, 64, A, A, A, None) == SHAPE
    assert L.mxfp8_gemm(A, 1, 16, 64, A, A + 1, A, None) == ALIGN
    # 32-bit buffer offsets: N * K and M * K * 2 must stay below 2^31
    assert L.mxfp8_gemm(A, 1, 1 << 20, 1 << 11, A, A, A, None) == SHAPE
    assert L.mxfp8_gemm(A, 1 << 19, 16, 1 << 11, A, A, A, None) == SHAPE


def test_last_error_empty_before_any_launch():
    assert M.lib().moe_last_error().decode() == ""


def test_router_logits_refusals():
    L = M.lib()
    assert L.moe_router_logits(None, A, 4, 64, 8, A, None) == NULL
    assert L.moe_router_logits(A, A, 4, 64, 8, None, None) == NULL
    assert L.moe_router_logits(A, A, 0, 64, 8, A, None) == SHAPE
    assert L.moe_router_logits(A, A, 4, 48, 8, A, None) == SHAPE
    assert L.moe_router_logits(A, A, 4, 64, 0, A, None) == SHAPE
    assert L.moe_router_logits(A, A, 4, 64, (1 << 20) + 1, A, None) == SHAPE
    # 32-bit buffer offsets: T * d * 2 and E * d * 2 must stay below 2^31
    assert L.moe_router_logits(A, A, 1 << 16, 1 << 14, 8, A, None) == SHAPE
    assert L.moe_router_logits(A, A, 4, 1 << 14, 1 << 16, A, None) == SHAPE
    assert L.moe_router_logits(A, A + 2, 4, 64, 8, A, None) == ALIGN


def test_route_policy_refusals():
    L = M.lib()
    ws = 0
    assert L.moe_route_topk_policy(None, 4, 8, 2, 0, None, A, A, A, A, A, None, ws, None) == NULL
    assert L.moe_route_topk_policy(A, 4, 8, 9, 0, None, A, A, A, A, A, None, ws, None) == SHAPE
    for bad in (-1, 4, 99):
        assert L.moe_route_topk_policy(A, 4, 8, 2, bad, None, A, A, A, A, A, None, ws, None) == 6
    assert L.moe_status_string(6).decode() == "MOE_E_POLICY"
    assert L.moe_route_topk_policy(A, 4, 8, 2, 2, A + 4, A, A, A, A, A, None, ws, None) == ALIGN


def test_combine_shared_refusals():
    L = M.lib()
    assert L.moe_combine_shared(A, A, A, 4, 2, 64, None, None, A, None) == NULL
    assert L.moe_combine_shared(None, A, A, 4, 2, 64, A, None, A, None) == NULL
    assert L.moe_combine_shared(A, A, A, 4, 33, 64, A, None, A, None) == SHAPE
    assert L.moe_combine_shared(A, A, A, 4, 2, 48, A, A, A, None) == SHAPE
    assert L.moe_combine_shared(A, A, A, 4, 2, 64, A + 4, None, A, None) == ALIGN
    assert L.moe_combine_shared(A, A, A, 4, 2, 64, A, A + 8, A, None) == ALIGN


def test_route_ffn_refusals():
    L = M.lib()
    ex = M._Experts(*([A] * 9))
    T, d, f, E, k = 4, 256, 128, 8, 2
    need = L.moe_expert_ffn_nvfp4_workspace(T, d, f, E, k)

    def call(lg=A, x=A, T=T, d=d, f=f, E=E, k=k, ids=A, w=A, off=A, sr=A, ro=A, y=A, ws=A, wsb=need):
        return L.moe_route_expert_ffn_nvfp4(lg, x, T, d, f, E, k, ctypes.byref(ex), ids, w, off, sr, ro, y, ws, wsb,
                                            None)
    assert call(lg=None) == NULL
    assert call(ro=None) == NULL
    assert call(x=None) == NULL
    # only the few-token path, E <= 256, k <= 16
    assert call(T=17, wsb=L.moe_expert_ffn_nvfp4_workspace(17, d, f, E, k)) == SHAPE
    assert call(E=257, wsb=L.moe_expert_ffn_nvfp4_workspace(T, d, f, 257, k)) == SHAPE
    assert call(E=64, k=17, wsb=L.moe_expert_ffn_nvfp4_workspace(T, d, f, 64, 17)) == SHAPE
    assert call(lg=A + 4) == ALIGN
    assert call(w=A + 8) == ALIGN
    assert call(ws=None) == WS



def test_layer_refusals():
    L = M.lib()
    ex = M._Experts(*([A] * 9))
    sx = M._Experts(*([A] * 9))
    T, d, f, E, k = 4, 256, 128, 8, 2
    need = L.moe_layer_nvfp4_workspace(T, d, f, E, k, 0)
    need_sh = L.moe_layer_nvfp4_workspace(T, d, f, E, k, 1)
    assert need_sh > need > 0
    assert L.moe_layer_nvfp4_workspace(17, d, f, E, k, 0) == 0  # more than 16 tokens
    assert L.moe_layer_nvfp4_workspace(T, d, f, 257, k, 0) == 0
    assert L.moe_layer_nvfp4_workspace(T, d, f, 64, 17, 0) == 0

    def call(lg=A, ld=0, x=A, T=T, d=d, f=f, E=E, k=k, sh=None, g=None, gld=1, res=None, ids=None, out=A, ws=A,
             wsb=None):
        if wsb is None:
            wsb = need_sh if sh is not None else need
        return L.moe_layer_nvfp4(lg, ld, x, T, d, f, E, k, ctypes.byref(ex), ctypes.byref(sh) if sh else None, g,
                                 gld, res, ids, None, None, None, None, out, ws, wsb, None)
    assert call(lg=None) == NULL
    assert call(x=None) == NULL
    assert call(out=None) == NULL
    assert call(ws=None) == NULL
    assert call(g=A) == NULL                     # a gate logit without a shared expert
    assert call(T=17) == SHAPE
    assert call(ld=E - 1) == SHAPE               # logits rows narrower than E
    assert call(sh=sx, g=A, gld=0) == SHAPE
    assert call(wsb=need - 1) == WS
    assert call(sh=sx, wsb=need) == WS           # the shared expert needs the larger workspace
    assert call(lg=A + 4) == ALIGN
    assert call(res=A + 2) == ALIGN
    assert call(ids=A + 4) == ALIGN


def test_ffn_autotune_refusals():
    L = M.lib()
    ex = M._Experts(*([A] * 9))
    T, d, f, E, k = 4, 256, 128, 8, 2
    need = L.moe_expert_ffn_nvfp4_workspace(T, d, f, E, k)

    def call(x=A, T=T, off=A, sr=A, reps=5, ws=A, wsb=need):
        return L.moe_ffn_autotune(x, T, d, f, E, k, ctypes.byref(ex), off, sr, A, ws, wsb, reps, None, None, None)
    assert call(off=None) == NULL
    assert call(x=None) == NULL
    assert call(T=17, wsb=L.moe_expert_ffn_nvfp4_workspace(17, d, f, E, k)) == SHAPE  # a batch: no pick
    assert call(reps=0) == SHAPE
    assert call(ws=None) == WS
    assert call(off=A + 4) == ALIGN
    assert M.STATUS_NAMES[L.moe_ffn_force_path(2)] == "MOE_E_SHAPE"
    assert L.moe_ffn_force_path(-1) == 0


def test_wait_limits_round_trip():
    """moe_set_wait_limits / moe_get_wait_limits (host state only, no GPU call)."""
    L = M.lib()
    prev = M.set_wait_limits(3, 7)
    assert M.wait_limits() == (3, 7)
    M.set_wait_limits(*prev)
    assert M.wait_limits() == prev == (256, 1 << 20)
    assert L.moe_status_string(7) == b"MOE_E_WAIT_EXPIRED"


def test_no_alloc_entry_refuses_beyond_its_scratch():
    """moe_expert_ffn_nvfp4_scratch refuses a shape whose H exceeds the static scratch
    (the long-prompt configuration needs 128 MiB) before any HIP call, naming the sizes;
    a refused shape is named as by the workspace entry point."""
    L = M.lib()
    ex = M._Experts(*([16] * 9))
    fake = 256  # aligned, never dereferenced: the refusal comes first
    st = L.moe_expert_ffn_nvfp4_scratch(fake, 4096, 7168, 2048, 256, 8, ctypes.byref(ex), fake, fake, fake, None)
    assert M.STATUS_NAMES[st] == "MOE_E_WORKSPACE"
    msg = L.moe_last_error().decode()
    assert "static scratch holds 33554432" in msg and str(M.expert_ffn_workspace(4096, 7168, 2048, 256, 8)) in msg
    assert M.expert_ffn_workspace(4096, 7168, 2048, 256, 8) > M.SCRATCH_BYTES
    st = L.moe_expert_ffn_nvfp4_scratch(fake, 4, 48, 32, 8, 2, ctypes.byref(ex), fake, fake, fake, None)
    assert M.STATUS_NAMES[st] == "MOE_E_SHAPE"


def test_combine_residual_refusals():
    L = M.lib()
    p = 256
    assert M.STATUS_NAMES[L.moe_combine_residual(p, p, p, 4, 2, 64, None, None, None, p, None)] == "MOE_E_NULL"
    assert M.STATUS_NAMES[L.moe_combine_residual(p, p, p, 4, 2, 64, None, p, p, p, None)] == "MOE_E_NULL"
    assert M.STATUS_NAMES[L.moe_combine_residual(p, p, p, 4, 2, 48, None, None, p, p, None)] == "MOE_E_SHAPE"
    assert M.STATUS_NAMES[L.moe_combine_residual(p, p, p, 4, 2, 64, None, None, p + 8, p, None)] == "MOE_E_ALIGN"


def test_mxfp8_pick_refusals():
    L = M.lib()
    p = 256
    assert M.STATUS_NAMES[L.mxfp8_autotune(p, 17, 64, 64, p, p, p, 5, None, None, None)] == "MOE_E_SHAPE"
    assert M.STATUS_NAMES[L.mxfp8_autotune(p, 4, 64, 48, p, p, p, 5, None, None, None)] == "MOE_E_SHAPE"
    assert M.STATUS_NAMES[L.mxfp8_autotune(None, 4, 64, 64, p, p, p, 5, None, None, None)] == "MOE_E_NULL"
    assert M.STATUS_NAMES[L.mxfp8_force_kernel(3)] == "MOE_E_SHAPE"
    assert L.mxfp8_force_kernel(-1) == 0
