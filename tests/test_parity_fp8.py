"""GPU parity of the FP8 (E4M3) expert path against the oracle, at reduced DeepSeek-V3 shapes.

Bars: routing bit-exact given the GPU's fp32 logits; the permuted rows' E4M3 codes and 1x128
scales bit-exact against the oracle's quantiser; y_perm and y within 6e-2 (relative Frobenius) of
the float64 oracle, which keeps the SwiGLU activation unrounded (reading R7 of the oracle); and
y_perm within 5e-3 of the oracle's steps with h also quantised in 1x128 blocks, which is what the
kernels compute (that tighter bar catches a wrong scale index that 6e-2 could hide).
"""

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import e4m3, moe
from tests.checks import check_permutation, rel_frobenius
from tests.gpu_oracle import TOL, TOL_GATES, TOL_LOGITS, host, routing_from_logits, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_FP8_H_ROUNDED = 5e-3


def _cfg(**over):
    return moe_inputs.CONFIGS["deepseek_v3_fp8_zipf"].replace(zipf_bias=False, **over)


SMALL_FP8 = {
    # several M tiles per busy expert, ragged last N tile of the second GEMM (640 = 2.5 x 256)
    "fp8_small": _cfg(T=300, H=640, E=16, k=4, F=384, Fs=256),
    # one K block in the second GEMM (F = 128), H = 384 (1.5 N tiles), tiny expert count
    "fp8_k128": _cfg(T=130, H=384, E=4, k=2, F=128, Fs=128),
    # k = E: every expert gets every token
    "fp8_all_experts": _cfg(T=70, H=256, E=4, k=4, F=256, Fs=0),
    # the API maxima: 512 experts (the largest tile-map prefix), top-16
    "fp8_api_maxima": _cfg(T=200, H=256, E=512, k=16, F=128, Fs=0),
}


def _skewed_bias(E):
    """Descending routing bias: a strongly uneven load, and the last expert never chosen."""
    b = torch.linspace(1.5, -1.5, E, dtype=torch.float32)
    if E > 4:
        b[-1] = -1.0e4
    return b.to(DEV)


def _make(cfg, seed=0):
    d = moe_inputs.make_inputs(cfg, seed=seed, weight_device=DEV, act_device=DEV)
    if cfg.k < cfg.E:
        d["bias"] = _skewed_bias(cfg.E)
    return d, moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)


def _h_rounded_expert(rows_hat, w1, w2):
    """Oracle steps of one expert with h quantised like the kernels: x_hat @ W1 -> SwiGLU -> 1x128 E4M3."""
    h = moe.swiglu_hidden(rows_hat, w1)
    codes, scales = e4m3.quantise_rows_1x128(h.astype(np.float32))
    return e4m3.dequantise_rows_1x128(codes, scales) @ w2


@pytest.mark.parametrize("name", sorted(SMALL_FP8))
def test_fp8_forward_matches_oracle(name):
    cfg = SMALL_FP8[name]
    print(f"[parity-fp8] forward {name}: {cfg}", flush=True)
    d, layer = _make(cfg)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    torch.cuda.synchronize()
    x = host(d["x"])
    w1 = [weights_of(d["w1"], d["w1_scales"], e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], d["w2_scales"], e) for e in range(cfg.E)]
    sw1 = weights_of(d["ws1"], d["ws1_scales"], None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], d["ws2_scales"], None) if cfg.Fs else None
    o = moe.forward(x, host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k,
                    score=cfg.score, norm=cfg.norm, bias=None if d["bias"] is None else host(d["bias"]),
                    shared_w1=sw1, shared_w2=sw2, fp8=True, logits=host(dbg["logits"]))
    # route + dispatch: bit-exact from the GPU's own logits
    assert rel_frobenius(host(dbg["logits"]), o["logits_oracle"]) <= TOL_LOGITS
    assert np.array_equal(host(dbg["topk_ids"]), o["ids"])
    assert rel_frobenius(host(dbg["topk_gates"]), o["gates"]) <= TOL_GATES
    for key, ref in (("expert_counts", "counts"), ("expert_offsets", "offsets"), ("row_map", "row_map"),
                     ("src_token", "src_token")):
        assert np.array_equal(host(dbg[key]), o[ref]), key
    check_permutation(o["ids"], o["counts"], o["offsets"], o["row_map"], o["src_token"])
    print(f"[parity-fp8] {name}: expert rows {o['counts'].tolist()}", flush=True)
    # quantised permuted rows: codes and scales bit-exact
    codes, scales = e4m3.quantise_rows_1x128(x)
    src = o["src_token"]
    assert np.array_equal(host(dbg["x_perm"]), codes[src])
    assert np.array_equal(host(dbg["x_perm_scales"]), scales[src])
    # experts: the oracle (h unrounded) and the oracle's steps with h rounded
    yp = host(dbg["y_perm"])
    e_yp = rel_frobenius(yp, o["y_perm"])
    e_y = rel_frobenius(host(y), o["y"])
    xp_hat = o["x_perm"]
    ref_hq = np.zeros_like(o["y_perm"])
    for e in range(cfg.E):
        a, b = int(o["offsets"][e]), int(o["offsets"][e + 1])
        if b > a:
            ref_hq[a:b] = _h_rounded_expert(xp_hat[a:b], w1[e], w2[e])
    e_hq = rel_frobenius(yp, ref_hq)
    print(f"[parity-fp8] {name}: rel_frob y_perm {e_yp:.3e} (h-rounded steps {e_hq:.3e})  y {e_y:.3e}",
          flush=True)
    assert e_yp <= TOL["fp8"] and e_y <= TOL["fp8"]
    assert e_hq <= TOL_FP8_H_ROUNDED


def test_fp8_stage_calls_match_oracle():
    """Per-stage entry points in FP8: quantising permute, then the grouped GEMMs on its output."""
    cfg = SMALL_FP8["fp8_small"]
    d, _ = _make(cfg)
    ids, gates, logits = moe_gpu.route(d["x"], d["w_router"], cfg.k, cfg.score, cfg.norm, d["bias"],
                                       return_logits=True)
    p = moe_gpu.permute(d["x"], ids, cfg.E, perm_dtype=torch.float8_e4m3fn)
    yp = moe_gpu.grouped_swiglu(p["x_perm"], p["offsets"], d["w1"], d["w2"], x_perm_scales=p["x_perm_scales"],
                                w1_scales=d["w1_scales"], w2_scales=d["w2_scales"])
    yp32 = moe_gpu.grouped_swiglu(p["x_perm"], p["offsets"], d["w1"], d["w2"], x_perm_scales=p["x_perm_scales"],
                                  w1_scales=d["w1_scales"], w2_scales=d["w2_scales"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    r = routing_from_logits(logits, d["bias"], cfg.k, cfg.score, cfg.norm, cfg.E)
    for key in ("offsets", "row_map", "src_token"):
        assert np.array_equal(host(p[key]), r[key]), key
    xp_hat = e4m3.dequantise_rows_1x128(host(p["x_perm"]), host(p["x_perm_scales"]))
    off = r["offsets"]
    w1 = [weights_of(d["w1"], d["w1_scales"], e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], d["w2_scales"], e) for e in range(cfg.E)]
    ref = moe.grouped_experts(xp_hat, off, lambda e: w1[e], lambda e: w2[e])
    assert rel_frobenius(host(yp), ref) <= TOL["fp8"]
    ref_hq = np.zeros_like(ref)
    for e in range(cfg.E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            ref_hq[a:b] = _h_rounded_expert(xp_hat[a:b], w1[e], w2[e])
    e32 = rel_frobenius(host(yp32), ref_hq)
    print(f"[parity-fp8] stage calls: fp32-output y_perm vs h-rounded steps {e32:.3e}", flush=True)
    assert e32 <= TOL_FP8_H_ROUNDED
    # the bf16 output is the fp32 one rounded once
    assert rel_frobenius(host(yp), host(yp32)) <= 4e-3


def test_fp8_dense_quantiser_via_single_expert_permute():
    """permute() with every token on expert 0 is the dense 1x128 quantiser in token order."""
    cfg = SMALL_FP8["fp8_k128"]
    d, _ = _make(cfg)
    ids = torch.zeros(cfg.T, 1, dtype=torch.int32, device=DEV)
    p = moe_gpu.permute(d["x"], ids, 1, perm_dtype=torch.float8_e4m3fn)
    torch.cuda.synchronize()
    codes, scales = e4m3.quantise_rows_1x128(host(d["x"]))
    assert np.array_equal(host(p["x_perm"]), codes)
    assert np.array_equal(host(p["x_perm_scales"]), scales)


def test_fp8_special_values_quantise_exactly():
    """Rows holding zeros, exact powers of two, values at rounding midpoints and a huge outlier."""
    H, T = 256, 8
    x = np.zeros((T, H), dtype=np.float32)
    x[1, :] = 1.0                                            # one value per block: scale 1/448
    x[2, :128] = np.float32(2.0) ** np.clip(np.arange(128) - 10, -10, 20)  # powers of two
    x[3, :] = np.linspace(-3.0, 3.0, H, dtype=np.float32)
    x[4, 0] = 3.0e4                                          # one outlier flattens its block
    x[4, 1:128] = 1.0e-3
    x[5, :] = -0.0
    x[6, ::2] = 1.0
    x[6, 1::2] = -(1.0 + 1.0 / 16.0)                         # midpoint between two codes after scaling
    x[7, :] = np.float32(448.0)
    xt = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    ids = torch.zeros(T, 1, dtype=torch.int32, device=DEV)
    p = moe_gpu.permute(xt, ids, 1, perm_dtype=torch.float8_e4m3fn)
    torch.cuda.synchronize()
    codes, scales = e4m3.quantise_rows_1x128(host(xt))
    assert np.array_equal(host(p["x_perm_scales"]), scales)
    assert np.array_equal(host(p["x_perm"]), codes)


@pytest.mark.parametrize("which", ["w1", "w2", "x"])
def test_fp8_arbitrary_block_scales(which):
    """Block scales that are not powers of two (one weight block, or the caller's activation
    scales) take the kernels' general path, which must match the oracle like the power-of-two one."""
    cfg = SMALL_FP8["fp8_small"]
    print(f"[parity-fp8] arbitrary scales in {which}", flush=True)
    d, _ = _make(cfg)
    ids, _, _ = moe_gpu.route(d["x"], d["w_router"], cfg.k, cfg.score, cfg.norm, d["bias"], return_logits=True)
    p = moe_gpu.permute(d["x"], ids, cfg.E, perm_dtype=torch.float8_e4m3fn)
    xs = p["x_perm_scales"].clone()
    w1s, w2s = d["w1_scales"].clone(), d["w2_scales"].clone()
    if which == "w1":
        w1s[cfg.E - 1, 1, 2] *= 1.1
    elif which == "w2":
        w2s[0, 2, 0] *= 0.7
    else:
        xs *= 1.3
    yp = moe_gpu.grouped_swiglu(p["x_perm"], p["offsets"], d["w1"], d["w2"], x_perm_scales=xs,
                                w1_scales=w1s, w2_scales=w2s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    off = host(p["offsets"])
    xp_hat = e4m3.dequantise_rows_1x128(host(p["x_perm"]), host(xs))
    ref_hq = np.zeros((xp_hat.shape[0], cfg.H))
    for e in range(cfg.E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            ref_hq[a:b] = _h_rounded_expert(xp_hat[a:b], weights_of(d["w1"], w1s, e), weights_of(d["w2"], w2s, e))
    err = rel_frobenius(host(yp), ref_hq)
    print(f"[parity-fp8] arbitrary scales in {which}: y_perm vs h-rounded steps {err:.3e}", flush=True)
    assert err <= TOL_FP8_H_ROUNDED
    if which != "x":  # the fused forward (rows gathered from x) on the same weights
        layer = moe_gpu.Layer.from_inputs(dict(d, w1_scales=w1s, w2_scales=w2s), cfg.k, cfg.score, cfg.norm)
        _, dbg = moe_gpu.forward(d["x"], layer, debug=True)
        torch.cuda.synchronize()
        assert np.array_equal(host(dbg["expert_offsets"]), off)
        err_f = rel_frobenius(host(dbg["y_perm"]), ref_hq)
        print(f"[parity-fp8] arbitrary scales in {which}: forward y_perm {err_f:.3e}", flush=True)
        assert err_f <= TOL_FP8_H_ROUNDED
