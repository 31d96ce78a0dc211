"""The seeded input generator: determinism, shapes, and the stored routing bias."""

import numpy as np
import torch

import moe_inputs
from oracle import moe


def test_deterministic_and_shaped():
    cfg = moe_inputs.CONFIGS["tiny_fp32"]
    a = moe_inputs.make_inputs(cfg, seed=0)
    b = moe_inputs.make_inputs(cfg, seed=0)
    c = moe_inputs.make_inputs(cfg, seed=1)
    for key in ("x", "w_router", "w1", "w2"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    assert a["x"].shape == (256, 128) and a["w_router"].shape == (128, 8)
    assert a["w1"].shape == (8, 128, 512) and a["w2"].shape == (8, 256, 128)
    assert abs(a["w_router"].std().item() - 0.02) < 0.002
    assert abs(a["w1"].std().item() - 128 ** -0.5) < 0.01


def test_fp8_weights_and_scales():
    cfg = moe_inputs.CONFIGS["deepseek_v3_fp8_zipf"].replace(T=4, H=256, E=3, F=128, Fs=128, zipf_bias=False)
    d = moe_inputs.make_inputs(cfg, seed=0)
    assert d["w1"].dtype == torch.float8_e4m3fn and d["w1_scales"].shape == (3, 2, 2)
    assert d["w2_scales"].shape == (3, 1, 2) and d["ws1_scales"].shape == (2, 2)
    # power-of-two block scales: each block's amax lands in the top binade (224, 448]
    q = d["w1"][0].float().reshape(2, 128, 2, 128).abs().amax(dim=(1, 3))
    assert (q >= 224.0).all() and (q <= 448.0).all()
    s = d["w1_scales"][0]
    m, _ = torch.frexp(s)
    assert (m == 0.5).all()


def test_tie_heavy_router_logits_are_exact():
    cfg = moe_inputs.CONFIGS["qwen3_235b"].replace(T=64)
    x, w = moe_inputs.tie_heavy_router(cfg)
    lg = moe.router_logits(x.float().numpy(), w.numpy())
    assert np.array_equal(lg * 8, np.round(lg * 8))
    ids = moe.topk_ids(lg, cfg.k)
    assert ids.shape == (64, 8)


def test_stored_zipf_bias_gives_zipf_loads():
    cfg = moe_inputs.CONFIGS["deepseek_v3_fp8_zipf"]
    b = moe_inputs.load_zipf_bias().numpy()
    assert b.shape == (256,) and b.dtype == np.float32
    assert (b == np.float32(-1e4)).sum() == 16
    x, w = moe_inputs.make_host_inputs(cfg, seed=0)
    lg = moe.router_logits(x.float().numpy(), w.numpy())
    load = moe.expert_counts(moe.topk_ids(moe.selection_key(lg, b), cfg.k), cfg.E)
    assert load.sum() == cfg.T * cfg.k and (load == 0).sum() == 16 and load.max() <= cfg.T
    s = np.sort(load)[::-1][2:240].astype(np.float64)
    slope = np.polyfit(np.log(np.arange(3, 241)), np.log(np.maximum(s, 1)), 1)[0]
    assert abs(slope + 1.2) < 0.2
