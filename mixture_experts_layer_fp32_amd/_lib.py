"""ctypes view of libmoe_mi355x.so (the C ABI in include/moe.h).  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

_c = ctypes
_vp, _i32, _i64, _sz = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_size_t

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_TOO_LARGE = range(6)
MOE_STATIC_SCRATCH_BYTES = 64 << 20
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2, 3
MOE_SOFTMAX, MOE_SIGMOID = 0, 1

# every function the header declares, with its argument and result types
SIGNATURES = {
    "moe_status_str": ([_i32], _c.c_char_p),
    "moe_abi_version": ([], _i32),
    "moe_route_workspace_size": ([_i64, _i32, _i32, _i32], _sz),
    "moe_route": ([_vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_permute_workspace_size": ([_i64, _i32, _i32], _sz),
    "moe_permute": ([_vp, _i32, _vp, _i64, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                     _vp], _i32),
    "moe_grouped_swiglu_workspace_size": ([_i64, _i32, _i32], _sz),
    "moe_grouped_swiglu": ([_vp, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                            _sz, _vp], _i32),
    "moe_unpermute_combine": ([_vp, _i32, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _i32, _vp], _i32),
    "moe_workspace_size": ([_vp, _i64], _sz),
    "moe_forward": ([_vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_backward_workspace_size": ([_vp, _i64], _sz),
    "moe_backward": ([_vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_forward_static": ([_vp, _vp, _i64, _vp, _vp, _vp], _i32),
}


class MoeLayerC(_c.Structure):
    """struct moe_layer."""
    _fields_ = [("H", _i32), ("E", _i32), ("k", _i32), ("F", _i32), ("Fs", _i32),
                ("x_dt", _i32), ("w_dt", _i32), ("out_dt", _i32), ("score", _i32), ("norm_topk", _i32),
                ("w_router", _vp), ("bias", _vp), ("w1", _vp), ("w2", _vp), ("ws1", _vp), ("ws2", _vp),
                ("w1_scales", _vp), ("w2_scales", _vp), ("ws1_scales", _vp), ("ws2_scales", _vp),
                ("gate_in_expert", _i32)]


class MoeDebugC(_c.Structure):
    """struct moe_debug."""
    _fields_ = [("logits", _vp), ("topk_ids", _vp), ("topk_gates", _vp), ("expert_counts", _vp),
                ("expert_offsets", _vp), ("row_map", _vp), ("src_token", _vp), ("x_perm", _vp),
                ("x_perm_scales", _vp), ("y_perm", _vp), ("stage_events", _vp * 7)]


MOE_NUM_BWD_STAGE_EVENTS = 9


class MoeRoutingC(_c.Structure):
    """struct moe_routing."""
    _fields_ = [("logits", _vp), ("topk_ids", _vp), ("topk_gates", _vp), ("expert_offsets", _vp),
                ("row_map", _vp), ("src_token", _vp)]


class MoeGradsC(_c.Structure):
    """struct moe_grads."""
    _fields_ = [("dx", _vp), ("dw_router", _vp), ("dw1", _vp), ("dw2", _vp), ("dws1", _vp), ("dws2", _vp)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {lib().moe_status_str(status).decode()}")
        self.status = status


_LIB = None


def lib():
    """Load the in-tree HIP library once; raise if it has not been built (there is no fallback)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_layer_fp32_amd.build`")
        handle = _c.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = handle
    return _LIB


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
