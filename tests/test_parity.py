"""GPU parity: the HIP path against the CPU oracle, stage by stage and end to end.

Bars: expert ids, counts, offsets, row_map, src_token and the permuted rows are bit-exact given
the GPU's own fp32 router logits; logits and gates within 1e-5 (relative Frobenius); y_perm and y
within 1e-5 (fp32), 2e-2 (bf16) of the float64 oracle.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import moe
from tests.checks import check_permutation, rel_frobenius
from tests.gpu_oracle import TOL, TOL_GATES, TOL_LOGITS, host, routing_from_logits, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _small(name, **over):
    return moe_inputs.CONFIGS[name].replace(**over)


# reduced shapes with the structure of each workload: several tiles and a ragged tail
SMALL = {
    "tiny_fp32": moe_inputs.CONFIGS["tiny_fp32"],
    "tiny_fp32_ragged": _small("tiny_fp32", T=97, E=6, k=3, H=96, F=160),
    "mixtral_small": _small("mixtral_8x7b", T=300, H=256, F=384),
    "qwen3_small": _small("qwen3_235b", T=333, H=320, E=16, k=4, F=256),
    "deepseek_small": _small("deepseek_v3", T=257, H=512, E=32, k=8, F=256, Fs=384),
    # experts averaging 192-288 rows: the 320-row GEMM tiles (two B stages; the second GEMM's
    # output staged per row group); H = 384 leaves a half N tile
    "deepseek_bm320": _small("deepseek_v3", T=520, H=384, E=8, k=4, F=256, Fs=256),
    # >= 768 rows per expert: the 256-row GEMM tiles; H not a multiple of 256 (ragged N tile)
    "mixtral_bigtile": _small("mixtral_8x7b", T=1700, H=320, E=3, k=2, F=384),
    # >= 64 experts: router logits through the dense GEMM kernel (3 x 96 columns: a ragged N tile)
    "qwen3_e96": _small("qwen3_235b", T=300, H=256, E=96, k=8, F=128),
    # few router tiles and a long H: the router GEMM splits K into 8 slices
    "qwen3_router_ksplit": _small("qwen3_235b", T=300, H=4096, E=64, k=8, F=128),
    # <= 16 experts, a long H and few tokens: the router cuts H over 4 (8) workgroup slices whose
    # partial logits the top-k kernel adds; T = 1000 leaves a partial last 64-token block
    "mixtral_router_4slices": _small("mixtral_8x7b", T=1000, H=2048, F=256),
    "mixtral_router_8slices": _small("mixtral_8x7b", T=200, H=4096, F=128),
    # <= 16 experts and >= 192 blocks of 16 tokens: the fused route kernel, with the three weight
    # parts packed as 1, 2 and 3 column tiles (E = 5, 8 and 16) and parts of two experts sharing a
    # tile (E = 6); softmax, sigmoid with selection bias, renormalised gates
    "fused_route_e8": _small("mixtral_8x7b", T=3100, H=256, F=128),
    "fused_route_e5_sigmoid": _small("deepseek_v3", T=3072 + 1, H=320, E=5, k=2, F=128, Fs=0),
    "fused_route_e16": _small("qwen3_235b", T=3200, H=512, E=16, k=4, F=128),
    "fused_route_e6": _small("mixtral_8x7b", T=3100, H=192, E=6, k=3, F=128),
}


def _dtype_key(cfg):
    return "fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype


def _make(cfg, seed=0):
    d = moe_inputs.make_inputs(cfg, seed=seed, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    return d, layer


def _oracle_layer(cfg, d, logits_gpu):
    """Full oracle forward (float64) on host copies, routing driven by the GPU logits."""
    w1 = [weights_of(d["w1"], d["w1_scales"], e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], d["w2_scales"], e) for e in range(cfg.E)]
    sw1 = weights_of(d["ws1"], d["ws1_scales"], None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], d["ws2_scales"], None) if cfg.Fs else None
    return moe.forward(host(d["x"]), host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], E=cfg.E,
                       k=cfg.k, score=cfg.score, norm=cfg.norm,
                       bias=None if d["bias"] is None else host(d["bias"]), shared_w1=sw1, shared_w2=sw2,
                       fp8=cfg.w_dtype == "fp8", logits=host(logits_gpu))


@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_matches_oracle(name):
    cfg = SMALL[name]
    print(f"[parity] forward {name}: {cfg}", flush=True)
    d, layer = _make(cfg)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    torch.cuda.synchronize()
    o = _oracle_layer(cfg, d, dbg["logits"])
    # route: logits within tolerance, ids/gates from the same fp32 logits
    assert rel_frobenius(host(dbg["logits"]), o["logits_oracle"]) <= TOL_LOGITS
    assert np.array_equal(host(dbg["topk_ids"]), o["ids"])
    assert rel_frobenius(host(dbg["topk_gates"]), o["gates"]) <= TOL_GATES
    # dispatch: bit-exact
    for key, ref in (("expert_counts", "counts"), ("expert_offsets", "offsets"), ("row_map", "row_map"),
                     ("src_token", "src_token")):
        assert np.array_equal(host(dbg[key]), o[ref]), key
    check_permutation(host(dbg["topk_ids"]), host(dbg["expert_counts"]), host(dbg["expert_offsets"]),
                      host(dbg["row_map"]), host(dbg["src_token"]))
    assert np.array_equal(host(dbg["x_perm"]), moe.permute_rows(host(d["x"]), o["src_token"]))
    # compute + combine
    tol = TOL[_dtype_key(cfg)]
    e_yp = rel_frobenius(host(dbg["y_perm"]), o["y_perm"])
    e_y = rel_frobenius(host(y), o["y"])
    print(f"[parity] {name}: rel_frob y_perm {e_yp:.3e}  y {e_y:.3e}  (tol {tol})", flush=True)
    assert e_yp <= tol and e_y <= tol


@pytest.mark.parametrize("name", ["tiny_fp32", "mixtral_small", "deepseek_small"])
def test_stage_calls_match_oracle(name):
    """The four per-stage entry points, each fed GPU outputs of the previous one."""
    cfg = SMALL[name]
    print(f"[parity] stages {name}", flush=True)
    d, _ = _make(cfg)
    ids, gates, logits = moe_gpu.route(d["x"], d["w_router"], cfg.k, cfg.score, cfg.norm, d["bias"],
                                       return_logits=True)
    ids2, gates2 = moe_gpu.route(d["x"], d["w_router"], cfg.k, cfg.score, cfg.norm, d["bias"])
    p = moe_gpu.permute(d["x"], ids, cfg.E)
    yp = moe_gpu.grouped_swiglu(p["x_perm"], p["offsets"], d["w1"], d["w2"])
    shared = None
    if cfg.Fs:
        off = torch.tensor([0, cfg.T], dtype=torch.int32, device=DEV)
        shared = moe_gpu.grouped_swiglu(d["x"], off, d["ws1"].unsqueeze(0), d["ws2"].unsqueeze(0))
    y = moe_gpu.unpermute_combine(yp, p["row_map"], gates, shared)
    torch.cuda.synchronize()
    r = routing_from_logits(logits, d["bias"], cfg.k, cfg.score, cfg.norm, cfg.E)
    assert torch.equal(ids, ids2) and torch.equal(gates, gates2)
    assert np.array_equal(host(ids), r["ids"])
    assert rel_frobenius(host(gates), r["gates"]) <= TOL_GATES
    for key in ("counts", "offsets", "row_map", "src_token"):
        assert np.array_equal(host(p[key]), r[key]), key
    # grouped GEMM on the GPU's permuted rows, expert by expert
    xp = host(p["x_perm"]).astype(np.float64)
    off = r["offsets"]
    ref_yp = moe.grouped_experts(xp, off, lambda e: weights_of(d["w1"], None, e),
                                 lambda e: weights_of(d["w2"], None, e))
    tol = TOL[_dtype_key(cfg)]
    assert rel_frobenius(host(yp), ref_yp) <= tol
    sh_ref = None
    if cfg.Fs:
        sh_ref = moe.swiglu_expert(host(d["x"]), weights_of(d["ws1"], None, None), weights_of(d["ws2"], None, None))
        assert rel_frobenius(host(shared), sh_ref) <= tol
    # combine on the GPU's own y_perm / gates / shared output: only the combine's rounding differs
    ref_y = moe.combine(host(yp), r["row_map"], host(gates), None if shared is None else host(shared))
    assert rel_frobenius(host(y), ref_y) <= (1e-6 if cfg.act_dtype == "f32" else 4e-3)


def test_identity_like_combine_returns_input():
    """Combine with y_perm := x_perm and normalised gates returns x (bf16: exactly up to one rounding)."""
    cfg = SMALL["qwen3_small"]
    d, _ = _make(cfg)
    ids, gates = moe_gpu.route(d["x"], d["w_router"], cfg.k, "sigmoid", True)
    p = moe_gpu.permute(d["x"], ids, cfg.E)
    y = moe_gpu.unpermute_combine(p["x_perm"], p["row_map"], gates, out_dtype=torch.float32)
    x = host(d["x"])
    err = np.abs(host(y) - x)
    assert (err <= 4 * np.spacing(np.abs(x).astype(np.float32)) + 1e-30).all()


def test_forward_is_deterministic():
    cfg = SMALL["deepseek_small"]
    d, layer = _make(cfg)
    a = moe_gpu.forward(d["x"], layer)
    b = moe_gpu.forward(d["x"], layer)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
