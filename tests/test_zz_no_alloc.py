"""moe_forward_static: the fused forward on the library's static device scratch, for callers
that cannot allocate.  Its output must equal moe_forward's (same kernels, so bit for bit) on two
calls in a row, the second with fewer tokens (the scratch keeps the first call's contents), the
call must not change the device's free memory, and a request past the static limit is refused."""

import ctypes

import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from mixture_experts_layer_fp32_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"

REDUCED = {
    "bf16": moe_inputs.CONFIGS["deepseek_v3"].replace(T=300, H=512, E=32, k=8, F=256, Fs=128),
    "e4m3": moe_inputs.CONFIGS["deepseek_v3_fp8_zipf"].replace(T=300, H=512, E=32, k=8, F=256, Fs=128,
                                                               zipf_bias=False),
    "fp32": moe_inputs.CONFIGS["tiny_fp32"],
    "mxfp4": moe_inputs.CONFIGS["deepseek_v3_mxfp4"].replace(T=300, H=512, E=32, k=8, F=256, Fs=256),
}


def _free_bytes():
    hip = ctypes.CDLL("libamdhip64.so.7")
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def _static(layer, x, y):
    c = layer.c_struct(x.dtype)
    return _lib.lib().moe_forward_static(ctypes.byref(c), ctypes.c_void_p(x.data_ptr()), x.shape[0],
                                         ctypes.c_void_p(y.data_ptr()), None,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _check(layer, x, label):
    y_ref = moe_gpu.forward(x, layer)
    y = torch.full_like(y_ref, float("nan"))
    torch.cuda.synchronize()
    assert _static(layer, x, y) == _lib.MOE_OK
    torch.cuda.synchronize()
    same = torch.equal(y, y_ref)
    print(f"[no-alloc] {label}: T={x.shape[0]} bit-identical to moe_forward: {same}", flush=True)
    assert same
    # the same call again: the device's free memory must not move (the first call on a device may
    # load the code object that holds the static array; later calls allocate nothing)
    y.fill_(float("nan"))
    torch.cuda.synchronize()
    free0 = _free_bytes()
    assert _static(layer, x, y) == _lib.MOE_OK
    torch.cuda.synchronize()
    assert _free_bytes() == free0, f"{label}: device free memory changed across the call"
    assert torch.equal(y, y_ref)


@pytest.mark.parametrize("dtype", sorted(REDUCED))
def test_static_forward_equals_workspace_forward(dtype):
    cfg = REDUCED[dtype]
    d = moe_inputs.make_inputs(cfg, seed=3, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    x = d["x"]
    _check(layer, x, f"{dtype} first call")
    _check(layer, x[: cfg.T // 3 + 1].contiguous(), f"{dtype} second, smaller call")


def test_static_forward_at_its_limit_on_the_deepseek_v3_shape():
    """The full DeepSeek-V3-shaped layer (22.6 GB of weights): 292 tokens fit the static scratch and
    match moe_forward; 293 are refused before anything is launched; then 40 tokens again."""
    cfg = moe_inputs.CONFIGS["deepseek_v3"]
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    _check(layer, d["x"][:292].contiguous(), "deepseek_v3 292 tokens")
    y = torch.empty(293, cfg.H, dtype=torch.bfloat16, device=DEV)
    assert _static(layer, d["x"][:293].contiguous(), y) == _lib.MOE_ERR_TOO_LARGE
    _check(layer, d["x"][1000:1040].contiguous(), "deepseek_v3 40 tokens")
