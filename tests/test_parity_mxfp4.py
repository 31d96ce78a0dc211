"""GPU parity of the MXFP4 expert path (both operands of both expert GEMMs 4-bit, E8M0 scales per 32
elements) against the oracle's MXFP4 mode (reading R8: x quantised per token and h per row in 1x32
blocks, the rest float64 on the dequantised operands).

Bars: routing and permutation bit-exact from the GPU's fp32 logits; the permuted rows' E2M1 codes
and E8M0 scales bit for bit against the oracle's quantiser (x is bf16, exact in fp32, so both sides
decide every code from the same value); y_perm and y within 2e-2 relative Frobenius error of the
oracle, and every row within 6e-2.  What separates the two sides is the accumulation order of u
(fp32 MFMA vs float64): an h element that lands within that difference of an E2M1 rounding
boundary can take the neighbouring code (one 4-bit step on one of F values), which moves its row
by about step / sqrt(F) -- a few per cent of that one row for the smallest F here -- and the bf16
rounding of the outputs (2^-9).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import moe, mxfp4
from tests.checks import check_permutation, max_row_rel, rel_frobenius
from tests.gpu_oracle import TOL, TOL_LOGITS, host, routing_from_logits, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_ROW = 6e-2


def _cfg(**over):
    return moe_inputs.CONFIGS["deepseek_v3_mxfp4"].replace(**over)


SMALL = {
    # several m-tiles per busy expert, shared expert, two N tiles in the second GEMM
    "mxfp4_small": _cfg(T=300, H=512, E=16, k=4, F=256, Fs=256),
    # long contraction (H = 2048: 8 K stages), one expert with most rows via a skewed bias
    "mxfp4_long_k": _cfg(T=200, H=2048, E=8, k=2, F=512, Fs=0, score="softmax", norm=False),
    # k = E: every expert gets every token
    "mxfp4_all_experts": _cfg(T=70, H=256, E=4, k=4, F=256, Fs=0),
    # the API maxima: 512 experts, top-16
    "mxfp4_api_maxima": _cfg(T=200, H=256, E=512, k=16, F=256, Fs=0),
}


def _check(label, got, ref):
    fro, row = rel_frobenius(got, ref), max_row_rel(got, ref)
    print(f"[mxfp4] {label}: rel_frob {fro:.3e}, worst row {row:.3e} ({len(ref)} rows)", flush=True)
    assert fro <= TOL["mxfp4"] and row <= TOL_ROW, label


@pytest.mark.parametrize("name", sorted(SMALL))
def test_mxfp4_forward_matches_oracle(name):
    cfg = SMALL[name]
    print(f"[mxfp4] {name}: {cfg}", flush=True)
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=DEV, act_device=DEV)
    if name == "mxfp4_long_k":
        d["bias"] = torch.linspace(2.0, -2.0, cfg.E, device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    torch.cuda.synchronize()
    w1 = [weights_of(d["w1"], d["w1_scales"], e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], d["w2_scales"], e) for e in range(cfg.E)]
    sw1 = weights_of(d["ws1"], d["ws1_scales"], None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], d["ws2_scales"], None) if cfg.Fs else None
    x = host(d["x"])
    o = moe.forward(x, host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k, score=cfg.score,
                    norm=cfg.norm, bias=None if d["bias"] is None else host(d["bias"]), shared_w1=sw1,
                    shared_w2=sw2, mxfp4_mode=True, logits=host(dbg["logits"]))
    assert rel_frobenius(host(dbg["logits"]), o["logits_oracle"]) <= TOL_LOGITS
    for key, ref in (("topk_ids", "ids"), ("expert_counts", "counts"), ("expert_offsets", "offsets"),
                     ("row_map", "row_map"), ("src_token", "src_token")):
        assert np.array_equal(host(dbg[key]), o[ref]), key
    check_permutation(o["ids"], o["counts"], o["offsets"], o["row_map"], o["src_token"])
    # permuted rows: E2M1 codes and E8M0 scales, bit for bit
    codes, scales = mxfp4.quantise_rows(x)
    assert np.array_equal(host(dbg["x_perm"]), mxfp4.pack(codes)[o["src_token"]])
    assert np.array_equal(host(dbg["x_perm_scales"]), scales[o["src_token"]])
    _check(f"{name} y_perm", host(dbg["y_perm"]), o["y_perm"])
    _check(f"{name} y", host(y), o["y"])


def test_mxfp4_stage_calls_match_the_fused_forward():
    """moe_permute (MXFP4 rows) + moe_grouped_swiglu + moe_unpermute_combine give the fused forward's
    y bit for bit (same kernels on the same codes)."""
    cfg = SMALL["mxfp4_small"]
    d = moe_inputs.make_inputs(cfg, seed=1, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    p = moe_gpu.permute(d["x"], dbg["topk_ids"], cfg.E, perm_dtype=moe_gpu.FP4)
    assert torch.equal(p["x_perm"].view(torch.uint8), dbg["x_perm"].view(torch.uint8))
    yp = moe_gpu.grouped_swiglu(p["x_perm"], p["offsets"], d["w1"], d["w2"], x_perm_scales=p["x_perm_scales"],
                                w1_scales=d["w1_scales"], w2_scales=d["w2_scales"])
    assert torch.equal(yp, dbg["y_perm"])
    off1 = torch.tensor([0, cfg.T], dtype=torch.int32, device=DEV)
    q = moe_gpu.permute(d["x"], torch.zeros(cfg.T, 1, dtype=torch.int32, device=DEV), 1, perm_dtype=moe_gpu.FP4)
    sh = moe_gpu.grouped_swiglu(q["x_perm"], off1, d["ws1"].unsqueeze(0), d["ws2"].unsqueeze(0),
                                x_perm_scales=q["x_perm_scales"], w1_scales=d["ws1_scales"].unsqueeze(0),
                                w2_scales=d["ws2_scales"].unsqueeze(0))
    y2 = moe_gpu.unpermute_combine(yp, p["row_map"], dbg["topk_gates"], shared=sh)
    torch.cuda.synchronize()
    assert torch.equal(y2, y)


def test_mxfp4_full_size_deepseek_v3():
    """The DeepSeek-V3-shaped layer with MXFP4 experts at full size, in bench.py's launch
    configuration: codes and scales of every permuted row bit-exact; y_perm on 8 rows of every expert
    and all rows of 256 sampled tokens, and y of those tokens against the oracle's MXFP4 layer."""
    cfg = moe_inputs.CONFIGS["deepseek_v3_mxfp4"]
    T, k, E = cfg.T, cfg.k, cfg.E
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, k, cfg.score, cfg.norm)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    torch.cuda.synchronize()
    x = host(d["x"])
    r = routing_from_logits(dbg["logits"], d["bias"], k, cfg.score, cfg.norm, E)
    assert np.array_equal(host(dbg["topk_ids"]), r["ids"])
    for key, ref in (("expert_offsets", "offsets"), ("row_map", "row_map"), ("src_token", "src_token")):
        assert np.array_equal(host(dbg[key]), r[ref]), key
    codes, scales = mxfp4.quantise_rows(x)
    src = r["src_token"]
    assert np.array_equal(host(dbg["x_perm"]), mxfp4.pack(codes)[src])
    assert np.array_equal(host(dbg["x_perm_scales"]), scales[src])
    x_in = mxfp4.dequantise_rows(codes, scales)
    del codes, scales
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(T, 256, replace=False))
    token_rows = r["row_map"][tokens]
    off = r["offsets"]
    picks = {}
    for e in np.nonzero(r["counts"])[0]:
        a, b = int(off[e]), int(off[e + 1])
        picks[int(e)] = set(rng.choice(np.arange(a, b), min(8, b - a), replace=False).tolist())
    for t_rows, t_ids in zip(token_rows, r["ids"][tokens]):
        for p, e in zip(t_rows, t_ids):
            picks[int(e)].add(int(p))

    def one_expert(e):
        p = np.array(sorted(picks[e]))
        return p, moe.swiglu_expert(x_in[src[p]], weights_of(d["w1"], d["w1_scales"], e),
                                    weights_of(d["w2"], d["w2_scales"], e), mxfp4.quantised)

    with ThreadPoolExecutor(8) as ex:
        results = list(ex.map(one_expert, sorted(picks)))
    rows = np.concatenate([p for p, _ in results])
    ref_rows = np.concatenate([ref for _, ref in results])
    _check(f"deepseek_v3_mxfp4 y_perm, {len(picks)} experts",
           host(dbg["y_perm"][torch.as_tensor(rows, device=DEV, dtype=torch.int64)]), ref_rows)
    ref_of = dict(zip(rows.tolist(), ref_rows))
    s_ref = moe.swiglu_expert(x_in[tokens], weights_of(d["ws1"], d["ws1_scales"], None),
                              weights_of(d["ws2"], d["ws2_scales"], None), mxfp4.quantised)
    yp_local = np.stack([ref_of[int(p)] for p in token_rows.ravel()])
    y_ref = moe.combine(yp_local, np.arange(256 * k).reshape(256, k), r["gates"][tokens], s_ref)
    _check("deepseek_v3_mxfp4 y of 256 tokens", host(y[torch.as_tensor(tokens, device=DEV)]), y_ref)
