"""GPU parity on seeded random layer shapes: every expert count, top-k, ragged token count and
tile shape the kernels accept, in bf16 and e4m3, with and without a shared expert and a
skewed routing bias.  Each case runs the fused forward and checks routing bit-exactly (from
the GPU's own logits) and the outputs against the float64 oracle within the dtype's bar.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import moe
from tests.checks import check_permutation, rel_frobenius
from tests.gpu_oracle import TOL, TOL_GATES, TOL_LOGITS, host, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 16


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    fp8 = bool(seed % 3 == 2)
    E = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 40, 64, 70]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([1, 7, 64, 129, 300, 513, 700]))
    H = int(rng.choice([128, 256, 384, 640] if fp8 else [64, 192, 256, 320, 512]))
    F = int(rng.choice([128, 256, 384]))
    Fs = int(rng.choice([0, 0, 128, 256]))
    score = "sigmoid" if rng.random() < 0.5 else "softmax"
    norm = bool(rng.random() < 0.5)
    base = moe_inputs.CONFIGS["deepseek_v3_fp8_zipf" if fp8 else "deepseek_v3"]
    cfg = base.replace(T=T, H=H, E=E, k=k, F=F, Fs=Fs, score=score, norm=norm, zipf_bias=False)
    skew = E > k and rng.random() < 0.5
    return cfg, skew


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_layer_matches_oracle(seed):
    cfg, skew = _case(seed)
    print(f"[parity-random] seed {seed}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F} Fs={cfg.Fs} "
          f"{cfg.score} norm={cfg.norm} w={cfg.w_dtype} skew={skew}", flush=True)
    d = moe_inputs.make_inputs(cfg, seed=seed, weight_device=DEV, act_device=DEV)
    if skew:
        d["bias"] = torch.linspace(2.0, -2.0, cfg.E, dtype=torch.float32, device=DEV)
    _check_layer(cfg, d, seed)


@pytest.mark.parametrize("w_dtype", ["bf16", "e4m3"])
def test_one_dominant_expert_matches_oracle(w_dtype):
    """One expert takes most rows (the grouped GEMMs' skewed-load tile map), the rest a few each."""
    base = moe_inputs.CONFIGS["deepseek_v3" if w_dtype == "bf16" else "deepseek_v3_fp8_zipf"]
    cfg = base.replace(T=2000, H=256, E=16, k=2, F=256, Fs=0, zipf_bias=False)
    d = moe_inputs.make_inputs(cfg, seed=5, weight_device=DEV, act_device=DEV)
    d["bias"] = torch.zeros(cfg.E, dtype=torch.float32, device=DEV)
    d["bias"][3] = 8.0
    print(f"[parity-random] dominant expert, {w_dtype}", flush=True)
    counts = _check_layer(cfg, d, "dominant")
    m_tiles = -(-counts // 192)  # 192- and 256-row tiles give the same verdict here
    assert m_tiles.max() * (m_tiles > 0).sum() > 3 * m_tiles.sum()


def _check_layer(cfg, d, seed):
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    torch.cuda.synchronize()
    fp8 = cfg.w_dtype == "fp8"
    w1 = [weights_of(d["w1"], d["w1_scales"], e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], d["w2_scales"], e) for e in range(cfg.E)]
    sw1 = weights_of(d["ws1"], d["ws1_scales"], None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], d["ws2_scales"], None) if cfg.Fs else None
    o = moe.forward(host(d["x"]), host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k,
                    score=cfg.score, norm=cfg.norm, bias=None if d["bias"] is None else host(d["bias"]),
                    shared_w1=sw1, shared_w2=sw2, fp8=fp8, logits=host(dbg["logits"]))
    assert rel_frobenius(host(dbg["logits"]), o["logits_oracle"]) <= TOL_LOGITS
    assert np.array_equal(host(dbg["topk_ids"]), o["ids"])
    assert rel_frobenius(host(dbg["topk_gates"]), o["gates"]) <= TOL_GATES
    for key, ref in (("expert_counts", "counts"), ("expert_offsets", "offsets"), ("row_map", "row_map"),
                     ("src_token", "src_token")):
        assert np.array_equal(host(dbg[key]), o[ref]), key
    check_permutation(o["ids"], o["counts"], o["offsets"], o["row_map"], o["src_token"])
    tol = TOL["fp8" if fp8 else cfg.act_dtype]
    e_yp = rel_frobenius(host(dbg["y_perm"]), o["y_perm"])
    e_y = rel_frobenius(host(y), o["y"])
    print(f"[parity-random] seed {seed}: rows {o['counts'].tolist()[:12]} rel_frob y_perm {e_yp:.3e} y {e_y:.3e}",
          flush=True)
    assert e_yp <= tol and e_y <= tol
    return o["counts"]
