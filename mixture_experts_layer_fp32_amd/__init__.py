"""Dropless MoE layer forward for AMD MI355X -- Python binding of the C ABI in include/moe.h.

Every stage runs in the HIP kernels of libmoe_mi355x.so; this module only allocates
outputs and workspaces with torch (device memory) and passes raw pointers plus the
current HIP stream.  There is no CPU or PyTorch fallback: calls fail if the library
is not built or a tensor is not on the GPU.

Stages (summary page of "Scalable Training of Mixture-of-Experts Models with
Megatron Core", "Method", first paragraph): ``route`` -> ``permute`` ->
``grouped_swiglu`` -> ``unpermute_combine``; ``forward`` runs all of them in one call.
"""

from __future__ import annotations

import dataclasses
import ctypes

import torch

from . import _lib
from ._lib import MoeError  # noqa: F401

__all__ = ["route", "permute", "grouped_swiglu", "unpermute_combine", "forward", "forward_static", "Layer",
           "workspace_size", "MoeError"]

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16, torch.float8_e4m3fn: _lib.MOE_FP8_E4M3,
       torch.float4_e2m1fn_x2: _lib.MOE_MXFP4}
FP4 = torch.float4_e2m1fn_x2  # two E2M1 elements per byte (MXFP4 codes)
E8M0 = torch.float8_e8m0fnu   # MXFP4 block scales


def _bytes(shape, dtype, device):
    """A tensor of a byte-sized dtype, allocated as uint8 (torch has no fill kernels for the 4-bit and
    E8M0 dtypes)."""
    return torch.empty(shape, dtype=torch.uint8, device=device).view(dtype)
_SCORE = {"softmax": _lib.MOE_SOFTMAX, "sigmoid": _lib.MOE_SIGMOID}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("MoE tensors must be on the GPU (no CPU path exists)")
            if not t.is_contiguous():
                raise ValueError("MoE tensors must be contiguous")


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def route(x, w_router, k, score="softmax", norm=False, bias=None, return_logits=False):
    """Router: fp32 projection, softmax/sigmoid, top-k.  Returns (ids int32 [T,k], gates fp32 [T,k][, logits])."""
    _need_gpu(x, w_router, bias)
    T, H = x.shape
    E = w_router.shape[1]
    dev = x.device
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    gates = torch.empty(T, k, dtype=torch.float32, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev) if return_logits else None
    L = _lib.lib()
    wsb = L.moe_route_workspace_size(T, H, E, int(return_logits))
    ws = _ws(wsb, dev)
    _lib.check("moe_route", L.moe_route(_ptr(x), _DT[x.dtype], _ptr(w_router), _ptr(bias), T, H, E, k,
                                        _SCORE[score], int(norm), _ptr(logits), _ptr(ids), _ptr(gates),
                                        _ptr(ws), wsb, _stream()))
    return (ids, gates, logits) if return_logits else (ids, gates)


def permute(x, ids, E, perm_dtype=None, with_rows=True):
    """Dispatch permutation.  Returns a dict: x_perm (+ x_perm_scales for fp8), row_map, src_token,
    counts, offsets (all int32 on the GPU)."""
    _need_gpu(x, ids)
    T, H = x.shape
    k = ids.shape[1]
    dev = x.device
    perm_dtype = perm_dtype or x.dtype
    R = T * k
    fp4 = perm_dtype == FP4
    out = {
        "row_map": torch.empty(T, k, dtype=torch.int32, device=dev),
        "src_token": torch.empty(R, dtype=torch.int32, device=dev),
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "x_perm": (None if not with_rows else _bytes((R, H // 2), FP4, dev) if fp4
                   else torch.empty(R, H, dtype=perm_dtype, device=dev)),
        "x_perm_scales": (_bytes((R, H // 32), E8M0, dev) if with_rows and fp4 else
                          torch.empty(R, H // 128, dtype=torch.float32, device=dev)
                          if with_rows and perm_dtype == torch.float8_e4m3fn else None),
    }
    L = _lib.lib()
    wsb = L.moe_permute_workspace_size(T, E, k)
    ws = _ws(wsb, dev)
    _lib.check("moe_permute", L.moe_permute(
        _ptr(x), _DT[x.dtype], _ptr(ids), T, H, E, k, _ptr(out["x_perm"]), _DT[perm_dtype],
        _ptr(out["x_perm_scales"]), _ptr(out["row_map"]), _ptr(out["src_token"]), _ptr(out["counts"]),
        _ptr(out["offsets"]), _ptr(ws), wsb, _stream()))
    return out


def grouped_swiglu(x_perm, offsets, w1, w2, x_perm_scales=None, w1_scales=None, w2_scales=None,
                   out_dtype=None):
    """All experts' SwiGLU MLPs over their contiguous rows (one grouped GEMM per matrix).  Returns y_perm."""
    _need_gpu(x_perm, offsets, w1, w2, x_perm_scales, w1_scales, w2_scales)
    rows, H = x_perm.shape
    if x_perm.dtype == FP4:  # contraction-contiguous MXFP4: x_perm [rows, H/2], w1 [E, 2F, H/2]
        H *= 2
        E, F2, _ = w1.shape
    else:
        E, _, F2 = w1.shape
    F = F2 // 2
    dt = _DT[x_perm.dtype]
    if out_dtype is None:
        out_dtype = torch.float32 if x_perm.dtype == torch.float32 else torch.bfloat16
    y = torch.empty(rows, H, dtype=out_dtype, device=x_perm.device)
    L = _lib.lib()
    wsb = L.moe_grouped_swiglu_workspace_size(rows, F, dt)
    ws = _ws(wsb, x_perm.device)
    _lib.check("moe_grouped_swiglu", L.moe_grouped_swiglu(
        _ptr(x_perm), _ptr(x_perm_scales), dt, _ptr(offsets), rows, E, H, F, _ptr(w1), _ptr(w1_scales),
        _ptr(w2), _ptr(w2_scales), _ptr(y), _DT[out_dtype], _ptr(ws), wsb, _stream()))
    return y


def unpermute_combine(y_perm, row_map, gates, shared=None, out_dtype=None):
    """y[t] = sum_j gates[t,j] * y_perm[row_map[t,j]] (+ shared[t])."""
    _need_gpu(y_perm, row_map, gates, shared)
    T, k = row_map.shape
    H = y_perm.shape[1]
    out_dtype = out_dtype or y_perm.dtype
    y = torch.empty(T, H, dtype=out_dtype, device=y_perm.device)
    L = _lib.lib()
    _lib.check("moe_unpermute_combine", L.moe_unpermute_combine(
        _ptr(y_perm), _DT[y_perm.dtype], _ptr(row_map), _ptr(gates), _ptr(shared), T, H, k, _ptr(y),
        _DT[out_dtype], _stream()))
    return y


@dataclasses.dataclass
class Layer:
    """Weights and switches of one MoE layer (all tensors on the GPU)."""
    w_router: torch.Tensor
    w1: torch.Tensor
    w2: torch.Tensor
    k: int
    score: str = "softmax"
    norm: bool = False
    bias: torch.Tensor | None = None
    ws1: torch.Tensor | None = None
    ws2: torch.Tensor | None = None
    w1_scales: torch.Tensor | None = None
    w2_scales: torch.Tensor | None = None
    ws1_scales: torch.Tensor | None = None
    ws2_scales: torch.Tensor | None = None
    out_dtype: torch.dtype | None = None
    gate_in_expert: bool = False  # fold the routing gate into the experts' SwiGLU epilogue

    @classmethod
    def from_inputs(cls, d: dict, k: int, score: str, norm: bool, out_dtype=None,
                    gate_in_expert: bool = False) -> "Layer":
        return cls(w_router=d["w_router"], w1=d["w1"], w2=d["w2"], k=k, score=score, norm=norm,
                   bias=d.get("bias"), ws1=d.get("ws1"), ws2=d.get("ws2"), w1_scales=d.get("w1_scales"),
                   w2_scales=d.get("w2_scales"), ws1_scales=d.get("ws1_scales"),
                   ws2_scales=d.get("ws2_scales"), out_dtype=out_dtype, gate_in_expert=gate_in_expert)

    def c_struct(self, x_dtype) -> _lib.MoeLayerC:
        H, E = self.w_router.shape
        if self.w1.dtype == FP4:  # w2 [E, H, F/2], ws2 [H, Fs/2]
            F = 2 * self.w2.shape[2]
            Fs = 0 if self.ws2 is None else 2 * self.ws2.shape[1]
        else:
            F = self.w2.shape[1]
            Fs = 0 if self.ws2 is None else self.ws2.shape[0]
        out_dt = self.out_dtype or x_dtype
        return _lib.MoeLayerC(
            H=H, E=E, k=self.k, F=F, Fs=Fs, x_dt=_DT[x_dtype], w_dt=_DT[self.w1.dtype], out_dt=_DT[out_dt],
            score=_SCORE[self.score], norm_topk=int(self.norm), w_router=self.w_router.data_ptr(),
            bias=None if self.bias is None else self.bias.data_ptr(), w1=self.w1.data_ptr(),
            w2=self.w2.data_ptr(), ws1=None if self.ws1 is None else self.ws1.data_ptr(),
            ws2=None if self.ws2 is None else self.ws2.data_ptr(),
            w1_scales=None if self.w1_scales is None else self.w1_scales.data_ptr(),
            w2_scales=None if self.w2_scales is None else self.w2_scales.data_ptr(),
            ws1_scales=None if self.ws1_scales is None else self.ws1_scales.data_ptr(),
            ws2_scales=None if self.ws2_scales is None else self.ws2_scales.data_ptr(),
            gate_in_expert=int(self.gate_in_expert))


def workspace_size(layer: Layer, T: int, x_dtype) -> int:
    c = layer.c_struct(x_dtype)
    return int(_lib.lib().moe_workspace_size(ctypes.byref(c), T))


def forward(x, layer: Layer, debug: bool = False, workspace=None):
    """The whole layer in one library call.  With debug=True also returns every intermediate."""
    tensors = [x, layer.w_router, layer.w1, layer.w2, layer.bias, layer.ws1, layer.ws2, layer.w1_scales,
               layer.w2_scales, layer.ws1_scales, layer.ws2_scales]
    _need_gpu(*tensors)
    T, H = x.shape
    E = layer.w_router.shape[1]
    k = layer.k
    dev = x.device
    c = layer.c_struct(x.dtype)
    out_dt = layer.out_dtype or x.dtype
    y = torch.empty(T, H, dtype=out_dt, device=dev)
    L = _lib.lib()
    need = int(L.moe_workspace_size(ctypes.byref(c), T))
    if need == 0 and T > 0:
        raise MoeError("moe_workspace_size", _lib.MOE_ERR_INVALID_ARG)
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, dev)
    dbg_c, dbg = None, None
    if debug:
        R = T * k
        fp8 = layer.w1.dtype == torch.float8_e4m3fn
        fp4 = layer.w1.dtype == FP4
        dbg = {
            "logits": torch.empty(T, E, dtype=torch.float32, device=dev),
            "topk_ids": torch.empty(T, k, dtype=torch.int32, device=dev),
            "topk_gates": torch.empty(T, k, dtype=torch.float32, device=dev),
            "expert_counts": torch.empty(E, dtype=torch.int32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "row_map": torch.empty(T, k, dtype=torch.int32, device=dev),
            "src_token": torch.empty(R, dtype=torch.int32, device=dev),
            "x_perm": _bytes((R, H // 2), FP4, dev) if fp4 else torch.empty(R, H, dtype=layer.w1.dtype, device=dev),
            "x_perm_scales": (torch.empty(R, H // 128, dtype=torch.float32, device=dev) if fp8 else
                              _bytes((R, H // 32), E8M0, dev) if fp4 else None),
            "y_perm": torch.empty(R, H, dtype=x.dtype, device=dev),
        }
        dbg_c = _lib.MoeDebugC(**{name: (None if t is None else t.data_ptr()) for name, t in dbg.items()})
    _lib.check("moe_forward", L.moe_forward(ctypes.byref(c), _ptr(x), T, _ptr(y),
                                            ctypes.byref(dbg_c) if dbg_c is not None else None,
                                            _ptr(workspace), workspace.numel(), _stream()))
    return (y, dbg) if debug else y


def forward_static(x, layer: Layer, out=None):
    """The whole layer on the library's static device scratch (moe_forward_static): no workspace is
    passed and the library allocates nothing; ``out`` ([T, H], optional) receives y.  Raises
    MoeError (MOE_ERR_TOO_LARGE) past the static limit."""
    _need_gpu(x, layer.w_router, layer.w1, layer.w2, layer.bias, layer.ws1, layer.ws2, out)
    T, H = x.shape
    c = layer.c_struct(x.dtype)
    y = out if out is not None else torch.empty(T, H, dtype=layer.out_dtype or x.dtype, device=x.device)
    _lib.check("moe_forward_static", _lib.lib().moe_forward_static(ctypes.byref(c), _ptr(x), T, _ptr(y), None,
                                                                    _stream()))
    return y


ROUTING_KEYS = ("logits", "topk_ids", "topk_gates", "expert_offsets", "row_map", "src_token")


def _check_backward_args(x, dy, layer: Layer, routing: dict):
    """The kernels read dy in x's dtype and index the routing tensors by T, k and E unchecked: a
    mismatch would make them read past the caller's buffers, so it is refused here."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H], got {tuple(x.shape)}")
    T, H = x.shape
    E = layer.w_router.shape[1]
    k = layer.k
    if dy.dtype != x.dtype or tuple(dy.shape) != (T, H):
        raise ValueError(f"dy must match x ({x.dtype}, {(T, H)}), got {dy.dtype}, {tuple(dy.shape)}")
    if dy.device != x.device:
        raise ValueError("dy must be on x's device")
    want = {"logits": (torch.float32, (T, E)), "topk_ids": (torch.int32, (T, k)),
            "topk_gates": (torch.float32, (T, k)), "expert_offsets": (torch.int32, (E + 1,)),
            "row_map": (torch.int32, (T, k)), "src_token": (torch.int32, (T * k,))}
    for key, (dt, shape) in want.items():
        t = routing.get(key)
        if t is None:
            raise ValueError(f"routing[{key!r}] is missing")
        if t.dtype != dt or tuple(t.shape) != shape:
            raise ValueError(f"routing[{key!r}] must be {dt} {shape} for T={T}, k={k}, E={E}; "
                             f"got {t.dtype} {tuple(t.shape)}")
        if t.device != x.device:
            raise ValueError(f"routing[{key!r}] must be on x's device")


def backward_workspace_size(layer: Layer, T: int, x_dtype) -> int:
    c = layer.c_struct(x_dtype)
    return int(_lib.lib().moe_backward_workspace_size(ctypes.byref(c), T))


def backward(x, dy, layer: Layer, routing: dict, workspace=None, stage_events=None):
    """Gradients of the layer for upstream gradient dy, in one library call.

    ``routing`` holds the forward's routing state as ``forward(..., debug=True)`` returns it
    (logits, topk_ids, topk_gates, expert_offsets, row_map, src_token).  Returns a dict with
    dx [T, H] (x's dtype) and fp32 dw_router [H, E], dw1 [E, H, 2F], dw2 [E, F, H] and, with a
    shared expert, dws1 [H, 2Fs] and dws2 [Fs, H].  ``stage_events``: None or a list of
    MOE_NUM_BWD_STAGE_EVENTS raw hipEvent_t handles (ctypes.c_void_p, int or None) recorded at
    the stage boundaries.
    """
    _check_backward_args(x, dy, layer, routing)
    rt = [routing[kk] for kk in ROUTING_KEYS]
    _need_gpu(x, dy, layer.w_router, layer.w1, layer.w2, layer.ws1, layer.ws2, *rt)
    T, H = x.shape
    E = layer.w_router.shape[1]
    F = layer.w2.shape[1]
    dev = x.device
    c = layer.c_struct(x.dtype)
    f32 = torch.float32
    g = {"dx": torch.empty(T, H, dtype=x.dtype, device=dev),
         "dw_router": torch.empty(H, E, dtype=f32, device=dev),
         "dw1": torch.empty(layer.w1.shape[0], H, 2 * F, dtype=f32, device=dev),
         "dw2": torch.empty(layer.w2.shape[0], F, H, dtype=f32, device=dev),
         "dws1": None if layer.ws1 is None else torch.empty(tuple(layer.ws1.shape), dtype=f32, device=dev),
         "dws2": None if layer.ws2 is None else torch.empty(tuple(layer.ws2.shape), dtype=f32, device=dev)}
    L = _lib.lib()
    need = int(L.moe_backward_workspace_size(ctypes.byref(c), T))
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, dev)
    r_c = _lib.MoeRoutingC(**{kk: t.data_ptr() for kk, t in zip(ROUTING_KEYS, rt)})
    g_c = _lib.MoeGradsC(**{kk: (None if t is None else t.data_ptr()) for kk, t in g.items()})
    ev_c = None
    if stage_events is not None:
        ev_c = (ctypes.c_void_p * _lib.MOE_NUM_BWD_STAGE_EVENTS)(
            *[ev.value if isinstance(ev, ctypes.c_void_p) else ev for ev in stage_events])
    _lib.check("moe_backward", L.moe_backward(ctypes.byref(c), _ptr(x), _ptr(dy), T, ctypes.byref(r_c),
                                              ctypes.byref(g_c), ev_c, _ptr(workspace), workspace.numel(),
                                              _stream()))
    return g
