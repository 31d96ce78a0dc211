"""Seeded synthetic inputs for the dropless MoE layer forward.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic, so both the CPU oracle and the HIP path can consume it.

The method's workloads are training runs of DeepSeek-V3, Qwen3-235B and
similar models on real data ("Scalable Training of Mixture-of-Experts Models
with Megatron Core", index page abstract and summary page "Results").  No
dataset or trained weights are used here: every tensor is drawn from a seeded
normal distribution with the shapes of those models' MoE layers.

Recipe (all workloads, seed 0 unless stated):

* ``x``      [T, H] ~ N(0, 1), drawn in fp32 on the host, cast (RNE) to the
             activation dtype;
* ``w_router`` [H, E] fp32 ~ N(0, std_r) (0.02 for the tiny layer, 1/sqrt(H)
             otherwise), drawn on the host right after ``x``;
* ``w1[e]``  [H, 2F] ~ N(0, 1/sqrt(H)), ``w2[e]`` [F, H] ~ N(0, 1/sqrt(F)),
             drawn expert by expert (w1 for all experts, then w2), then the
             shared expert ``ws1`` [H, 2Fs], ``ws2`` [Fs, H], from a second
             generator seeded with seed + 1 on ``weight_device``;
* FP8 workloads: each weight matrix is drawn in fp32 as above and stored as
  E4M3 codes with one fp32 scale per 128x128 block (scale = the smallest power
  of two 2^q with 448 * 2^q >= the block's amax, 1 for an all-zero block;
  codes by torch's own float8_e4m3fn cast of w / scale after clamping to +-448);
* MXFP4 workloads: each weight matrix is drawn in fp32 as above, stored
  contraction-contiguous (W1[e] as [2F, H/2] bytes, W2[e] as [H, F/2]) as E2M1
  codes, two per byte (element 2i in the low nibble), with one E8M0 scale per
  32 consecutive elements along the contraction (the smallest power of two
  2^q with 6 * 2^q >= the block's amax; codes: nearest E2M1 value of w / 2^q,
  ties to the even-mantissa code), as torch float4_e2m1fn_x2 / float8_e8m0fnu;
* the skewed-routing workload adds a per-expert routing bias read from
  ``tests/golden/zipf_bias_deepseek_v3_fp8.txt`` (written by
  ``tests/golden/make_zipf_bias.py``), calibrated so expert loads follow a Zipf
  law with exponent 1.2 and 16 experts receive no tokens.
"""

from __future__ import annotations

import dataclasses
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
ZIPF_BIAS_FILE = os.path.join(os.path.dirname(_HERE), "tests", "golden", "zipf_bias_deepseek_v3_fp8.txt")


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    F: int
    Fs: int = 0
    score: str = "softmax"        # "softmax" | "sigmoid"
    norm: bool = False            # renormalise the k gates
    act_dtype: str = "f32"        # x / y dtype: "f32" | "bf16"
    w_dtype: str = "f32"          # expert weight dtype: "f32" | "bf16" | "fp8"
    router_std: float | None = None   # None: 1/sqrt(H)
    zipf_bias: bool = False
    description: str = ""

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def R(self) -> int:
        return self.T * self.k


CONFIGS = {
    "tiny_fp32": LayerConfig(
        "tiny_fp32", T=256, H=128, E=8, k=2, F=256, score="softmax", norm=False,
        act_dtype="f32", w_dtype="f32", router_std=0.02,
        description="tiny dropless MoE layer, all fp32: T=256 H=128 E=8 top-2 F=256"),
    "mixtral_8x7b": LayerConfig(
        "mixtral_8x7b", T=4096, H=4096, E=8, k=2, F=14336, score="softmax", norm=False,
        act_dtype="bf16", w_dtype="bf16",
        description="Mixtral-8x7B-shaped layer: T=4096 H=4096 E=8 top-2 F=14336, bf16, fp32 router"),
    "qwen3_235b": LayerConfig(
        "qwen3_235b", T=8192, H=4096, E=128, k=8, F=1536, score="softmax", norm=True,
        act_dtype="bf16", w_dtype="bf16",
        description="Qwen3-235B-shaped layer: T=8192 H=4096 E=128 top-8 F=1536, renormalised softmax"),
    "deepseek_v3": LayerConfig(
        "deepseek_v3", T=8192, H=7168, E=256, k=8, F=2048, Fs=2048, score="sigmoid", norm=True,
        act_dtype="bf16", w_dtype="bf16",
        description="DeepSeek-V3-shaped layer: T=8192 H=7168 E=256 top-8 F=2048 + shared expert, sigmoid"),
    "deepseek_v3_mxfp4": LayerConfig(
        "deepseek_v3_mxfp4", T=8192, H=7168, E=256, k=8, F=2048, Fs=2048, score="sigmoid", norm=True,
        act_dtype="bf16", w_dtype="mxfp4",
        description="DeepSeek-V3-shaped layer with MXFP4 expert GEMMs (E2M1, E8M0 per 32), bf16 activations"),
    "deepseek_v3_fp8_zipf": LayerConfig(
        "deepseek_v3_fp8_zipf", T=8192, H=7168, E=256, k=8, F=2048, Fs=2048, score="sigmoid",
        norm=True, act_dtype="bf16", w_dtype="fp8", zipf_bias=True,
        description="DeepSeek-V3-shaped layer with Zipf(1.2) expert loads and e4m3 expert GEMMs"),
}

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def load_zipf_bias(path: str = ZIPF_BIAS_FILE) -> torch.Tensor:
    """The stored routing bias (one fp32 per expert, written as hex floats)."""
    vals = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float.fromhex(line))
    return torch.tensor(vals, dtype=torch.float32)


def make_host_inputs(cfg: LayerConfig, seed: int = 0):
    """x (activation dtype) and w_router (fp32), drawn on the host in that order."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(cfg.T, cfg.H, generator=g, dtype=torch.float32).to(_TORCH_DT[cfg.act_dtype])
    std = cfg.router_std if cfg.router_std is not None else 1.0 / math.sqrt(cfg.H)
    w_router = torch.randn(cfg.H, cfg.E, generator=g, dtype=torch.float32) * std
    return x, w_router


def _block_fp8(w: torch.Tensor):
    """fp32 [K, N] -> (float8_e4m3fn codes [K, N], fp32 scales [K/128, N/128]); input preparation only.

    Scale of a 128x128 block: the smallest power of two 2^q with 448 * 2^q >= its amax.
    """
    K, N = w.shape
    wb = w.reshape(K // 128, 128, N // 128, 128)
    amax = wb.abs().amax(dim=(1, 3))
    m, e = torch.frexp(amax)
    q = (e - 9 + (m > 0.875).to(e.dtype)).clamp(-127, 127)
    s = torch.where(amax > 0, torch.ldexp(torch.ones_like(amax), q), torch.ones_like(amax))
    q = (wb / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(K, N), s.contiguous()


_FP4_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)  # between consecutive E2M1 magnitudes


def _mx_fp4(w: torch.Tensor):
    """fp32 [K, N] -> (E2M1 codes stored [N, K/2] as float4_e2m1fn_x2, E8M0 scales [N, K/32] as
    float8_e8m0fnu); input preparation only."""
    wt = w.t().contiguous()
    N, K = wt.shape
    b = wt.reshape(N, K // 32, 32)
    amax = b.abs().amax(dim=2)
    # smallest q with 6 * 2^q >= amax: from frexp(amax) = m * 2^e (m in [0.5, 1)), q = e - 2 - (m <= 0.75)
    m, e = torch.frexp(amax)
    q = (e - 2 - (m <= 0.75).to(e.dtype)).clamp(-127, 127)
    q = torch.where(amax > 0, q, torch.zeros_like(q))
    v = b * torch.ldexp(torch.ones_like(amax), -q)[:, :, None]
    mag = v.abs().clamp(max=6.0)
    code = torch.zeros_like(mag, dtype=torch.uint8)
    for i, mid in enumerate(_FP4_MIDS):  # ties: down at odd steps 0, 2, 4, 6 (strict), up at 1, 3, 5
        code += (mag > mid if i % 2 == 0 else mag >= mid).to(torch.uint8)
    code = torch.where((v < 0) & (code != 0), code | 8, code).reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed.view(torch.float4_e2m1fn_x2), (q + 127).to(torch.uint8).view(torch.float8_e8m0fnu)


def _draw_matrix(g, rows, cols, std, w_dtype, device):
    w = torch.randn(rows, cols, generator=g, dtype=torch.float32, device=device) * std
    if w_dtype == "fp8":
        return _block_fp8(w)
    if w_dtype == "mxfp4":
        return _mx_fp4(w)
    return w.to(_TORCH_DT[w_dtype]), None


def make_inputs(cfg: LayerConfig, seed: int = 0, weight_device: str = "cpu", act_device: str | None = None):
    """All layer inputs as torch tensors (dict).

    Keys: x, w_router, bias (or None), w1 [E,H,2F], w2 [E,F,H], w1_scales, w2_scales
    (fp8 only, else None), ws1, ws2, ws1_scales, ws2_scales (shared expert, or None).
    ``act_device`` defaults to ``weight_device``.
    """
    act_device = act_device or weight_device
    x, w_router = make_host_inputs(cfg, seed)
    bias = load_zipf_bias() if cfg.zipf_bias else None
    if bias is not None and bias.numel() != cfg.E:
        raise ValueError(f"stored bias has {bias.numel()} entries, layer has E={cfg.E}")
    gw = torch.Generator(device=weight_device).manual_seed(seed + 1)
    E, H, F, Fs = cfg.E, cfg.H, cfg.F, cfg.Fs
    fp8 = cfg.w_dtype == "fp8"
    fp4 = cfg.w_dtype == "mxfp4"
    if fp4:
        u8, e8 = torch.uint8, torch.float8_e8m0fnu
        w1 = torch.empty(E, 2 * F, H // 2, dtype=u8, device=weight_device).view(torch.float4_e2m1fn_x2)
        w2 = torch.empty(E, H, F // 2, dtype=u8, device=weight_device).view(torch.float4_e2m1fn_x2)
        w1s = torch.empty(E, 2 * F, H // 32, dtype=u8, device=weight_device).view(e8)
        w2s = torch.empty(E, H, F // 32, dtype=u8, device=weight_device).view(e8)
    else:
        wdt = torch.float8_e4m3fn if fp8 else _TORCH_DT[cfg.w_dtype]
        w1 = torch.empty(E, H, 2 * F, dtype=wdt, device=weight_device)
        w2 = torch.empty(E, F, H, dtype=wdt, device=weight_device)
        w1s = torch.empty(E, H // 128, 2 * F // 128, device=weight_device) if fp8 else None
        w2s = torch.empty(E, F // 128, H // 128, device=weight_device) if fp8 else None

    def put(dst, src):  # byte copy (torch has no copy kernels for the 4-bit / E8M0 dtypes)
        dst.view(torch.uint8).copy_(src.view(torch.uint8)) if fp4 else dst.copy_(src)

    for e in range(E):
        q, s = _draw_matrix(gw, H, 2 * F, 1.0 / math.sqrt(H), cfg.w_dtype, weight_device)
        put(w1[e], q)
        if fp8 or fp4:
            put(w1s[e], s)
    for e in range(E):
        q, s = _draw_matrix(gw, F, H, 1.0 / math.sqrt(F), cfg.w_dtype, weight_device)
        put(w2[e], q)
        if fp8 or fp4:
            put(w2s[e], s)
    ws1 = ws2 = ws1s = ws2s = None
    if Fs:
        ws1, ws1s = _draw_matrix(gw, H, 2 * Fs, 1.0 / math.sqrt(H), cfg.w_dtype, weight_device)
        ws2, ws2s = _draw_matrix(gw, Fs, H, 1.0 / math.sqrt(Fs), cfg.w_dtype, weight_device)
    return {
        "x": x.to(act_device), "w_router": w_router.to(act_device),
        "bias": None if bias is None else bias.to(act_device),
        "w1": w1, "w2": w2, "w1_scales": w1s, "w2_scales": w2s,
        "ws1": ws1, "ws2": ws2, "ws1_scales": ws1s, "ws2_scales": ws2s,
    }


def make_upstream_grad(cfg: LayerConfig, seed: int = 0, device: str = "cpu", T: int | None = None) -> torch.Tensor:
    """dL/dy for the backward: [T, H] standard normal (its own generator, seed + 2), in the
    activation dtype."""
    g = torch.Generator(device="cpu").manual_seed(seed + 2)
    T = cfg.T if T is None else T
    dy = torch.randn(T, cfg.H, generator=g, dtype=torch.float32)
    return dy.to(_TORCH_DT[cfg.act_dtype]).to(device)


def tie_heavy_router(cfg: LayerConfig, seed: int = 0):
    """Integer-valued x in {-2..2} and W_r in {-1, 0, 1}/8: router logits are exact multiples of
    1/8 in any summation order, so many keys tie exactly.  Returns (x, w_router) on the host."""
    g = torch.Generator(device="cpu").manual_seed(seed + 17)
    x = torch.randint(-2, 3, (cfg.T, cfg.H), generator=g).to(torch.float32).to(_TORCH_DT[cfg.act_dtype])
    w = torch.randint(-1, 2, (cfg.H, cfg.E), generator=g).to(torch.float32) / 8.0
    return x, w
