"""GPU parity of the layer backward (moe_backward) against the oracle's float64 chain rule.

The oracle backward (oracle/backward.py, pinned by finite differences) runs on the routing the
GPU forward chose (its fp32 logits), so both sides differentiate the same selection.  Bars
(relative Frobenius error of every gradient): 1e-5 with fp32 operands, 2e-2 with bf16 operands,
the forward's bars.  The fp32 path rounds only in fp32 (measured errors about 5e-7); the bf16
path also rounds du and g h to bf16 before their GEMMs (2^-9 relative per element; measured
about 2e-3).
"""

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import backward as obw
from oracle import moe
from tests.checks import rel_frobenius
from tests.gpu_oracle import host, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BWD = {"f32": 1e-5, "bf16": 2e-2}


def _cfg(name, **over):
    return moe_inputs.CONFIGS[name].replace(**over)


CASES = {
    "tiny_fp32": moe_inputs.CONFIGS["tiny_fp32"],
    # fp32, 5 experts (K = E = 5 and N = E = 5 in the router GEMMs: chunk tails), sigmoid, no norm
    "fp32_e5_sigmoid": _cfg("tiny_fp32", T=77, H=96, E=5, k=2, F=64, score="sigmoid", norm=False),
    # fp32 with a shared expert and renormalised sigmoid gates (96-wide ragged tiles)
    "fp32_shared_sigmoid": _cfg("tiny_fp32", T=150, H=96, E=6, k=3, F=96, Fs=64, score="sigmoid",
                                     norm=True),
    "mixtral_small": _cfg("mixtral_8x7b", T=300, H=256, F=384),
    "qwen3_small": _cfg("qwen3_235b", T=333, H=320, E=16, k=4, F=256),
    "deepseek_small": _cfg("deepseek_v3", T=257, H=512, E=32, k=8, F=256, Fs=384),
    # bf16 router products as split bf16 products (E % 32 == 0, H % 64 == 0) over 2 row slices of dW_r's
    # contraction (T >= 2048), a slice boundary inside a 64-row block
    "router_split_slices": _cfg("deepseek_v3", T=2100, H=256, E=32, k=2, F=128, Fs=128),
    # experts averaging 192-288 rows: the 320-row tiles in the recomputation and the data-gradient
    # products (fp32 results staged 32 rows at a time; dx_perm in bf16); H = 384 leaves a half N tile
    "deepseek_bm320": _cfg("deepseek_v3", T=520, H=384, E=8, k=4, F=256, Fs=256),
    # >= 128 rows per expert and H, 2F not multiples of 128: ragged M, N and K tiles everywhere
    "mixtral_ragged": _cfg("mixtral_8x7b", T=700, H=320, E=3, k=2, F=384),
    # most experts without rows: their weight gradients must be exactly zero
    "empty_experts": _cfg("qwen3_235b", T=5, H=128, E=64, k=2, F=128),
    # more than 8 output m-tiles in the weight-gradient GEMMs, a count not a multiple of 8 (the
    # grouped TN tile order walks groups of 8 m-tiles n-major; its last group is narrower):
    # bf16 256-row tiles, dW1 over H = 2368 (10 m-tiles) and dW2 over F = 2432 (10 m-tiles)
    "bf16_multi_group": _cfg("mixtral_8x7b", T=64, H=2368, E=4, k=2, F=2432),
    # fp32 128-row tiles, dW1 over H = 1184 (10 m-tiles), dW2 over F = 1152 (9 m-tiles)
    "fp32_multi_group": _cfg("tiny_fp32", T=40, H=1184, E=3, k=2, F=1152),
}


def run_case(cfg, seed=0):
    d = moe_inputs.make_inputs(cfg, seed=seed, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    x = d["x"]
    _, dbg = moe_gpu.forward(x, layer, debug=True)
    dy = moe_inputs.make_upstream_grad(cfg, seed=seed, device=DEV)
    g = moe_gpu.backward(x, dy, layer, dbg)
    torch.cuda.synchronize()
    w1 = [weights_of(d["w1"], None, e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], None, e) for e in range(cfg.E)]
    sw1 = weights_of(d["ws1"], None, None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], None, None) if cfg.Fs else None
    fw = moe.forward(host(x), host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k,
                     score=cfg.score, norm=cfg.norm, bias=None if d["bias"] is None else host(d["bias"]),
                     shared_w1=sw1, shared_w2=sw2, logits=host(dbg["logits"]))
    assert np.array_equal(host(dbg["topk_ids"]), fw["ids"])
    o = obw.backward(fw, host(x), host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], host(dy),
                     score=cfg.score, norm=cfg.norm, shared_w1=sw1, shared_w2=sw2)
    return g, o, fw


def errors(g, o):
    names = ["dx", "dw_router", "dw1", "dw2"] + (["dws1", "dws2"] if o["dws1"] is not None else [])
    return {n: rel_frobenius(host(g[n]), o[n]) for n in names}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    cfg = CASES[name]
    g, o, fw = run_case(cfg)
    err = errors(g, o)
    print(name, {k: f"{v:.2e}" for k, v in err.items()}, flush=True)
    tol = TOL_BWD[cfg.act_dtype]
    assert all(v <= tol for v in err.values()), err
    if name == "empty_experts":
        empty = np.flatnonzero(np.diff(fw["offsets"]) == 0)
        assert len(empty) >= cfg.E - 2 * cfg.T
        assert not host(g["dw1"])[empty].any() and not host(g["dw2"])[empty].any()


def test_backward_without_tokens_zeroes_weight_gradients():
    cfg = _cfg("deepseek_v3", T=0, H=128, E=8, k=2, F=128, Fs=128)
    d = moe_inputs.make_inputs(cfg.replace(T=1), seed=0, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    x = d["x"][:0]
    _, dbg = moe_gpu.forward(x, layer, debug=True)
    g = moe_gpu.backward(x, torch.empty_like(x), layer, dbg)
    torch.cuda.synchronize()
    for n in ("dw_router", "dw1", "dw2", "dws1", "dws2"):
        assert g[n].numel() > 0 and not g[n].any(), n
    assert g["dx"].shape == (0, cfg.H)


def test_backward_is_deterministic():
    cfg = CASES["qwen3_small"]
    d = moe_inputs.make_inputs(cfg, seed=1, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    _, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    dy = moe_inputs.make_upstream_grad(cfg, seed=1, device=DEV)
    a = moe_gpu.backward(d["x"], dy, layer, dbg)
    b = moe_gpu.backward(d["x"], dy, layer, dbg)
    torch.cuda.synchronize()
    for n in ("dx", "dw_router", "dw1", "dw2"):
        assert torch.equal(a[n], b[n]), n


def test_backward_hip_graph_capture_and_replay():
    """moe_backward records into a HIP graph (no sync, no allocation, no memset inside) and every
    replay, with eager work in between, reproduces the eager gradients bit for bit (the layer has
    a shared expert and a router gradient cut into row slices)."""
    cfg = CASES["deepseek_small"]
    d = moe_inputs.make_inputs(cfg, seed=2, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    x = d["x"]
    _, dbg = moe_gpu.forward(x, layer, debug=True)
    dy = moe_inputs.make_upstream_grad(cfg, seed=2, device=DEV)
    ws = torch.empty(moe_gpu.backward_workspace_size(layer, cfg.T, x.dtype), dtype=torch.uint8, device=DEV)
    eager = {n: t.clone() for n, t in moe_gpu.backward(x, dy, layer, dbg, workspace=ws).items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe_gpu.backward(x, dy, layer, dbg, workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = moe_gpu.backward(x, dy, layer, dbg, workspace=ws)
    for rep in range(3):
        junk = torch.randn(1000, 1000, device=DEV) @ torch.randn(1000, 1000, device=DEV)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in eager.items():
            assert torch.equal(out[n], t), f"replay {rep}: {n}"
        del junk
