"""The C ABI: the library loads, exports every function include/moe.h declares, and rejects bad
arguments on the host before launching anything (these calls never reach the GPU)."""

import ctypes
import os
import re

import pytest

from mixture_experts_layer_fp32_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

INVALID, UNSUP, WS = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED, _lib.MOE_ERR_WORKSPACE
P = ctypes.c_void_p(16 * 1024)  # a fake, 16-byte aligned "device" address: never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert len(names) == 14
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 2
    for s in range(6):
        assert L.moe_status_str(s).startswith(b"MOE_")


def _route(L, **over):
    a = dict(x=P, x_dt=1, w=P, bias=None, T=8, H=64, E=8, k=2, score=0, norm=0, logits=P, ids=P,
             gates=P, ws=P, wsb=1 << 20)
    a.update(over)
    return L.moe_route(a["x"], a["x_dt"], a["w"], a["bias"], a["T"], a["H"], a["E"], a["k"], a["score"],
                       a["norm"], a["logits"], a["ids"], a["gates"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(x=None), INVALID), (dict(ids=None), INVALID), (dict(k=0), INVALID), (dict(k=9), INVALID),
    (dict(E=513, k=2), INVALID), (dict(E=32, k=17), INVALID), (dict(H=12), INVALID), (dict(T=-1), INVALID),
    (dict(x_dt=2), INVALID), (dict(score=7), INVALID), (dict(ws=None), WS), (dict(logits=None, wsb=1024), WS),
    (dict(T=2 ** 30, k=2), INVALID)])
def test_route_rejects(over, code):
    assert _route(_lib.lib(), **over) == code


def test_route_with_no_tokens_is_a_noop():
    assert _route(_lib.lib(), T=0) == _lib.MOE_OK


def test_workspace_sizes():
    L = _lib.lib()
    assert L.moe_route_workspace_size(100, 64, 8, 1) >= 3 * 16 * 64 * 2
    assert L.moe_route_workspace_size(100, 64, 8, 0) >= 100 * 8 * 4 + 3 * 16 * 64 * 2
    assert L.moe_permute_workspace_size(1000, 64, 4) >= 1000 * 4 * 4
    assert L.moe_grouped_swiglu_workspace_size(512, 256, _lib.MOE_BF16) >= 512 * 256 * 2
    assert L.moe_grouped_swiglu_workspace_size(512, 256, _lib.MOE_F32) >= 512 * 256 * 4
    assert L.moe_grouped_swiglu_workspace_size(512, 256, _lib.MOE_FP8_E4M3) >= 512 * 256 + 512 * 2 * 4


def _permute(L, **over):
    a = dict(x=P, x_dt=1, ids=P, T=64, H=128, E=8, k=2, xp=P, pdt=1, sc=None, rm=P, src=P, cnt=None,
             off=P, ws=P, wsb=1 << 20)
    a.update(over)
    return L.moe_permute(a["x"], a["x_dt"], a["ids"], a["T"], a["H"], a["E"], a["k"], a["xp"], a["pdt"],
                         a["sc"], a["rm"], a["src"], a["cnt"], a["off"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(ids=None), INVALID), (dict(off=None), INVALID), (dict(pdt=0), INVALID),
    (dict(pdt=2), INVALID), (dict(pdt=2, sc=P, H=64), INVALID), (dict(x_dt=0, pdt=2, sc=P), INVALID),
    (dict(ws=None), WS), (dict(wsb=16), WS), (dict(x=ctypes.c_void_p(16 * 1024 + 4)), INVALID),
    (dict(T=0), UNSUP)])
def test_permute_rejects(over, code):
    assert _permute(_lib.lib(), **over) == code


def _gemm(L, **over):
    a = dict(xp=P, sc=None, dt=1, off=P, rows=128, E=4, H=256, F=256, w1=P, w1s=None, w2=P, w2s=None,
             y=P, odt=1, ws=P, wsb=1 << 30)
    a.update(over)
    return L.moe_grouped_swiglu(a["xp"], a["sc"], a["dt"], a["off"], a["rows"], a["E"], a["H"], a["F"],
                                a["w1"], a["w1s"], a["w2"], a["w2s"], a["y"], a["odt"], a["ws"], a["wsb"],
                                None)


@pytest.mark.parametrize("over,code", [
    (dict(off=None), INVALID), (dict(F=192), INVALID), (dict(H=96), INVALID), (dict(dt=0, odt=1), INVALID),
    (dict(dt=2), INVALID), (dict(dt=2, sc=P, w1s=P, w2s=P, H=192), INVALID), (dict(E=0), INVALID),
    (dict(E=600), INVALID), (dict(odt=2), INVALID), (dict(wsb=1024), WS), (dict(rows=0), _lib.MOE_OK),
    (dict(rows=0, xp=None, y=None), _lib.MOE_OK), (dict(xp=ctypes.c_void_p(16 * 1024 + 4)), INVALID),
    (dict(y=ctypes.c_void_p(16 * 1024 + 8), odt=0), INVALID)])
def test_grouped_swiglu_rejects(over, code):
    assert _gemm(_lib.lib(), **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(k=0), INVALID), (dict(H=12), INVALID), (dict(y=None), INVALID), (dict(ydt=2), INVALID),
    (dict(shared=ctypes.c_void_p(16 * 1024 + 8)), INVALID), (dict(T=0), _lib.MOE_OK)])
def test_combine_rejects(over, code):
    a = dict(yp=P, ydt=1, rm=P, g=P, shared=None, T=16, H=64, k=2, y=P, odt=1)
    a.update(over)
    L = _lib.lib()
    assert L.moe_unpermute_combine(a["yp"], a["ydt"], a["rm"], a["g"], a["shared"], a["T"], a["H"], a["k"],
                                   a["y"], a["odt"], None) == code


def _layer(**over):
    f = dict(H=256, E=8, k=2, F=256, Fs=0, x_dt=1, w_dt=1, out_dt=1, score=0, norm_topk=0, w_router=16384,
             bias=None, w1=16384, w2=16384, ws1=None, ws2=None, w1_scales=None, w2_scales=None,
             ws1_scales=None, ws2_scales=None)
    f.update(over)
    return _lib.MoeLayerC(**f)


@pytest.mark.parametrize("over", [dict(k=9), dict(w_dt=0), dict(x_dt=2), dict(F=100), dict(Fs=256),
                                  dict(w_dt=2), dict(w1=None), dict(score=3), dict(Fs=-1), dict(gate_in_expert=2),
                                  dict(w_dt=3), dict(w_dt=3, w1_scales=16384, w2_scales=16384, F=384),
                                  dict(w_dt=3, w1_scales=16384, w2_scales=16384, H=384), dict(w_dt=4)])
def test_forward_rejects_bad_layers(over):
    L = _lib.lib()
    lay = _layer(**over)
    assert L.moe_workspace_size(ctypes.byref(lay), 64) == 0
    assert L.moe_forward(ctypes.byref(lay), P, 64, P, None, P, 1 << 30, None) == INVALID


def test_mxfp4_layers_need_their_scales_and_have_no_backward():
    L = _lib.lib()
    lay = _layer(w_dt=3, w1_scales=16384, w2_scales=16384)
    need = L.moe_workspace_size(ctypes.byref(lay), 64)
    assert need > 0
    assert L.moe_backward_workspace_size(ctypes.byref(lay), 64) == 0
    assert L.moe_backward(ctypes.byref(lay), P, P, 64, None, None, None, P, 1 << 30, None) == UNSUP


def test_gate_in_expert_needs_a_per_row_gate_buffer():
    """Folding the gate into the experts carves one fp32 gate per permuted row from the workspace."""
    L = _lib.lib()
    plain = L.moe_workspace_size(ctypes.byref(_layer()), 64)
    folded = L.moe_workspace_size(ctypes.byref(_layer(gate_in_expert=1)), 64)
    assert folded - plain == 64 * 2 * 4 + (256 - 64 * 2 * 4 % 256) % 256


def test_forward_workspace_checks():
    L = _lib.lib()
    lay = _layer()
    need = L.moe_workspace_size(ctypes.byref(lay), 64)
    assert need > 64 * 256 * 2 * 2
    assert L.moe_forward(ctypes.byref(lay), P, 64, P, None, P, need - 1, None) == WS
    assert L.moe_forward(ctypes.byref(lay), P, 64, P, None, None, need, None) == WS
    assert L.moe_forward(ctypes.byref(lay), P, 0, P, None, P, need, None) == _lib.MOE_OK
    assert L.moe_forward(None, P, 64, P, None, P, need, None) == INVALID


def test_forward_checks_requested_debug_rows():
    """moe_forward writes x_perm only on request; e4m3 rows need their scales with them."""
    L = _lib.lib()
    lay = _layer(w_dt=2, w1_scales=16384, w2_scales=16384)
    need = L.moe_workspace_size(ctypes.byref(lay), 64)
    assert need > 0
    dbg = _lib.MoeDebugC()
    dbg.x_perm = 16 * 1024
    assert L.moe_forward(ctypes.byref(lay), P, 64, P, ctypes.byref(dbg), P, need, None) == INVALID
    dbg2 = _lib.MoeDebugC()
    dbg2.x_perm = 16 * 1024 + 2
    lay16 = _layer()
    need16 = L.moe_workspace_size(ctypes.byref(lay16), 64)
    assert L.moe_forward(ctypes.byref(lay16), P, 64, P, ctypes.byref(dbg2), P, need16, None) == INVALID


def _grads(**over):
    f = dict(dx=16384, dw_router=16384, dw1=16384, dw2=16384, dws1=None, dws2=None)
    f.update(over)
    return _lib.MoeGradsC(**f)


def _routing(**over):
    f = dict(logits=16384, topk_ids=16384, topk_gates=16384, expert_offsets=16384, row_map=16384, src_token=16384)
    f.update(over)
    return _lib.MoeRoutingC(**f)


def test_backward_workspace_size():
    """u, dh' (fp32), du (bf16, 64 zero rows after its end), g h (bf16), dg, dx_perm (bf16), dlogits
    and the router's dx term; with bf16 also the weight-gradient products' padded contraction tables, one
    transposed activation [max(H, F)][ld] (ld = rows + 64 E rounded up to 64) and dy in row order
    (+ 64 rows); each piece 256-byte aligned."""
    L = _lib.lib()
    lay = _layer()
    T, H, E, k, F = 64, 256, 8, 2, 256
    R = T * k

    def a(n):
        return (n + 255) // 256 * 256
    ld = (R + 64 * E + 63) // 64 * 64
    want = (a(R * 2 * F * 4) + a(R * F * 4) + a((R + 64) * 2 * F * 2) + a(R * F * 2) + a(R * 4) + a(R * H * 2)
            + a(T * E * 4) + a(T * H * 4) + a(2 * (E + 1) * 4) + a(16) + a(max(H, F) * ld * 2)
            + a((R + 64) * H * 2))
    assert L.moe_backward_workspace_size(ctypes.byref(lay), T) == want
    assert L.moe_backward_workspace_size(ctypes.byref(_layer(w_dt=2, w1_scales=16384, w2_scales=16384)), T) == 0
    assert L.moe_backward_workspace_size(ctypes.byref(_layer(k=9)), T) == 0


def test_backward_workspace_size_split_router():
    """bf16 layers with E % 32 == 0 and H % 64 == 0 take the router's products as split bf16 products:
    dlogits in three bf16 parts [T, 6E] and [T + 64, 3E], W_r's parts [H, 6E], the partial products of
    S = clamp(T // 1024, 1, 6) row slices [S, H, 3E] (fp32) and their offsets, in place of the fp32
    slices; the rest as above."""
    L = _lib.lib()
    T, H, E, k, F = 2048, 256, 64, 2, 256
    lay = _layer(E=E)
    R = T * k
    S = 2

    def a(n):
        return (n + 255) // 256 * 256
    ld = (R + 64 * E + 63) // 64 * 64
    want = (a(T * 6 * E * 2) + a(H * 6 * E * 2) + a((T + 64) * 3 * E * 2) + a(S * H * 3 * E * 4) + a((S + 1) * 4)
            + a(R * 2 * F * 4) + a(R * F * 4) + a((R + 64) * 2 * F * 2) + a(R * F * 2) + a(R * 4) + a(R * H * 2)
            + a(T * E * 4) + a(T * H * 4) + a(2 * (E + 1) * 4) + a(16) + a(max(H, F) * ld * 2)
            + a((R + 64) * H * 2))
    assert L.moe_backward_workspace_size(ctypes.byref(lay), T) == want


@pytest.mark.parametrize("case,code", [
    ("fp8", UNSUP), ("no_grads", INVALID), ("no_dw1", INVALID), ("misaligned_dx", INVALID),
    ("no_routing", INVALID), ("no_offsets", INVALID), ("shared_without_dws", INVALID),
    ("small_workspace", WS), ("no_workspace", WS), ("bad_layer", INVALID)])
def test_backward_rejects(case, code):
    L = _lib.lib()
    lay = _layer()
    r, g, ws = ctypes.byref(_routing()), ctypes.byref(_grads()), 1 << 30
    wsp = P
    if case == "fp8":
        lay = _layer(w_dt=2, w1_scales=16384, w2_scales=16384)
    elif case == "no_grads":
        g = None
    elif case == "no_dw1":
        g = ctypes.byref(_grads(dw1=None))
    elif case == "misaligned_dx":
        g = ctypes.byref(_grads(dx=16384 + 4))
    elif case == "no_routing":
        r = None
    elif case == "no_offsets":
        r = ctypes.byref(_routing(expert_offsets=None))
    elif case == "shared_without_dws":
        lay = _layer(Fs=256, ws1=16384, ws2=16384)
    elif case == "small_workspace":
        ws = L.moe_backward_workspace_size(ctypes.byref(lay), 64) - 1
    elif case == "no_workspace":
        wsp = None
    elif case == "bad_layer":
        lay = _layer(F=100)
    assert L.moe_backward(ctypes.byref(lay), P, P, 64, r, g, None, wsp, ws, None) == code


def test_forward_static_rejects_on_the_host():
    """moe_forward_static checks the layer and its scratch need before touching the device: a
    DeepSeek-V3-shaped layer fits MOE_STATIC_SCRATCH_BYTES up to 292 tokens, not 293."""
    L = _lib.lib()
    c = _lib.MoeLayerC(H=7168, E=256, k=8, F=2048, Fs=2048, x_dt=_lib.MOE_BF16, w_dt=_lib.MOE_BF16,
                       out_dt=_lib.MOE_BF16, score=_lib.MOE_SIGMOID, norm_topk=1, w_router=16, bias=None, w1=16,
                       w2=16, ws1=16, ws2=16, w1_scales=None, w2_scales=None, ws1_scales=None, ws2_scales=None)
    assert L.moe_workspace_size(ctypes.byref(c), 292) <= _lib.MOE_STATIC_SCRATCH_BYTES
    assert L.moe_workspace_size(ctypes.byref(c), 293) > _lib.MOE_STATIC_SCRATCH_BYTES
    assert L.moe_forward_static(ctypes.byref(c), P, 293, P, None, None) == _lib.MOE_ERR_TOO_LARGE
    assert L.moe_forward_static(ctypes.byref(c), P, 0, P, None, None) == _lib.MOE_OK
    assert L.moe_forward_static(None, P, 8, P, None, None) == INVALID
    c.k = 0
    assert L.moe_forward_static(ctypes.byref(c), P, 8, P, None, None) == INVALID


def _bwd_args(T=6, H=64, E=4, k=2, F=128, dt=None):
    import torch
    import mixture_experts_layer_fp32_amd as moe_gpu
    dt = dt or torch.bfloat16
    layer = moe_gpu.Layer(w_router=torch.zeros(H, E), w1=torch.zeros(E, H, 2 * F, dtype=dt),
                          w2=torch.zeros(E, F, H, dtype=dt), k=k)
    x = torch.zeros(T, H, dtype=dt)
    i32, f32 = torch.int32, torch.float32
    routing = {"logits": torch.zeros(T, E, dtype=f32), "topk_ids": torch.zeros(T, k, dtype=i32),
               "topk_gates": torch.zeros(T, k, dtype=f32), "expert_offsets": torch.zeros(E + 1, dtype=i32),
               "row_map": torch.zeros(T, k, dtype=i32), "src_token": torch.zeros(T * k, dtype=i32)}
    return x, torch.zeros_like(x), layer, routing


@pytest.mark.parametrize("bad", ["dy_dtype", "dy_shape", "logits", "topk_ids_dtype", "topk_gates", "offsets",
                                 "row_map", "src_token", "missing"])
def test_backward_binding_rejects_mismatched_tensors(bad):
    """The binding refuses, before any device call, a dy or routing state that does not match x, k
    and E (the kernels would read past the caller's buffers)."""
    import torch
    import mixture_experts_layer_fp32_amd as moe_gpu
    x, dy, layer, r = _bwd_args()
    T, H = x.shape
    if bad == "dy_dtype":
        dy = dy.float()
    elif bad == "dy_shape":
        dy = torch.zeros(T + 1, H, dtype=x.dtype)
    elif bad == "logits":
        r["logits"] = torch.zeros(T, 5)
    elif bad == "topk_ids_dtype":
        r["topk_ids"] = r["topk_ids"].long()
    elif bad == "topk_gates":
        r["topk_gates"] = torch.zeros(T, 3)
    elif bad == "offsets":
        r["expert_offsets"] = torch.zeros(4, dtype=torch.int32)
    elif bad == "row_map":
        r["row_map"] = torch.zeros(T - 1, 2, dtype=torch.int32)
    elif bad == "src_token":
        r["src_token"] = torch.zeros(T, dtype=torch.int32)
    elif bad == "missing":
        del r["row_map"]
    with pytest.raises(ValueError):
        moe_gpu.backward(x, dy, layer, r)


def test_backward_binding_accepts_matching_tensors_up_to_the_device_check():
    """Matching host tensors pass the shape checks and stop at the device check (no CPU path)."""
    import mixture_experts_layer_fp32_amd as moe_gpu
    x, dy, layer, r = _bwd_args()
    with pytest.raises(ValueError, match="GPU"):
        moe_gpu.backward(x, dy, layer, r)
