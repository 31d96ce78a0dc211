"""GPU parity at the full workload sizes, on every token where the oracle can afford it.

Per workload (seed 0): router logits vs the float64 oracle on all tokens; expert ids, gates,
counts, offsets, row_map and src_token from the GPU's own logits (bit-exact, all tokens);
permuted rows exact (all rows); expert outputs on every row of three sampled experts (the
busiest, the least busy non-empty one and one drawn at random); combine on all tokens from the
GPU's own expert outputs; the shared expert on sampled tokens.  In FP8 the permuted rows are
compared as E4M3 codes + 1x128 scales against the oracle's quantiser, bit for bit.
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


def _tol(cfg):
    return TOL["fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype]


@pytest.mark.parametrize("name", ["mixtral_8x7b", "qwen3_235b", "deepseek_v3", "deepseek_v3_fp8_zipf"])
def test_full_size_layer(name):
    cfg = moe_inputs.CONFIGS[name]
    print(f"[parity-full] {name}: {cfg.description}", flush=True)
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    torch.cuda.synchronize()
    x = host(d["x"])
    # route
    lg_o = moe.router_logits(x, host(d["w_router"]))
    lg_g = host(dbg["logits"])
    assert rel_frobenius(lg_g, lg_o) <= TOL_LOGITS
    r = routing_from_logits(dbg["logits"], d["bias"], cfg.k, cfg.score, cfg.norm, cfg.E)
    assert np.array_equal(host(dbg["topk_ids"]), r["ids"])
    assert rel_frobenius(host(dbg["topk_gates"]), r["gates"]) <= TOL_GATES
    agree = (moe.topk_ids(moe.selection_key(lg_o, None if d["bias"] is None else host(d["bias"])), cfg.k) ==
             r["ids"]).all(axis=1).mean()
    print(f"[parity-full] {name}: tokens whose ids match the oracle's own logits: {agree:.5f}", flush=True)
    # dispatch
    for key, ref in (("expert_counts", "counts"), ("expert_offsets", "offsets"), ("row_map", "row_map"),
                     ("src_token", "src_token")):
        assert np.array_equal(host(dbg[key]), r[ref]), key
    check_permutation(r["ids"], r["counts"], r["offsets"], r["row_map"], r["src_token"])
    fp8 = cfg.w_dtype == "fp8"
    if fp8:  # E4M3 codes and 1x128 scales of every permuted row, bit-exact
        codes, scales = e4m3.quantise_rows_1x128(x)
        assert np.array_equal(host(dbg["x_perm"]), codes[r["src_token"]])
        assert np.array_equal(host(dbg["x_perm_scales"]), scales[r["src_token"]])
        x_hat = e4m3.dequantise_rows_1x128(codes, scales)
        del codes, scales

        def rows_of(a, b):
            return x_hat[r["src_token"][a:b]]
    else:
        xp = host(dbg["x_perm"])
        assert np.array_equal(xp, x[r["src_token"]])

        def rows_of(a, b):
            return xp[a:b]
    # experts: every row of three sampled experts
    cnt, off = r["counts"], r["offsets"]
    nonzero = np.nonzero(cnt)[0]
    rng = np.random.default_rng(0)
    picks = sorted({int(np.argmax(cnt)), int(nonzero[np.argmin(cnt[nonzero])]), int(rng.choice(nonzero))})
    yp = dbg["y_perm"]
    errs = []
    for e in picks:
        a, b = int(off[e]), int(off[e + 1])
        ref = moe.swiglu_expert(rows_of(a, b), weights_of(d["w1"], d["w1_scales"], e), weights_of(d["w2"], d["w2_scales"], e))
        errs.append(rel_frobenius(host(yp[a:b]), ref))
    print(f"[parity-full] {name}: experts {picks} rows {[int(cnt[e]) for e in picks]} rel_frob {errs}", flush=True)
    assert max(errs) <= _tol(cfg)
    # shared expert on sampled tokens, then combine on all tokens from the GPU's own y_perm
    shared = None
    if cfg.Fs:
        sel = rng.choice(cfg.T, 64, replace=False)
        off1 = torch.tensor([0, cfg.T], dtype=torch.int32, device=DEV)
        if fp8:  # every token on one expert: permute() is the dense 1x128 quantiser
            xs = e4m3.dequantise_rows_1x128(*e4m3.quantise_rows_1x128(x[sel]))
            s_ref = moe.swiglu_expert(xs, weights_of(d["ws1"], d["ws1_scales"], None),
                                      weights_of(d["ws2"], d["ws2_scales"], None))
            q = moe_gpu.permute(d["x"], torch.zeros(cfg.T, 1, dtype=torch.int32, device=DEV), 1,
                                perm_dtype=torch.float8_e4m3fn)
            s_gpu = moe_gpu.grouped_swiglu(q["x_perm"], off1, d["ws1"].unsqueeze(0), d["ws2"].unsqueeze(0),
                                           x_perm_scales=q["x_perm_scales"],
                                           w1_scales=d["ws1_scales"].unsqueeze(0),
                                           w2_scales=d["ws2_scales"].unsqueeze(0))
        else:
            s_ref = moe.swiglu_expert(x[sel], weights_of(d["ws1"], d["ws1_scales"], None),
                                      weights_of(d["ws2"], d["ws2_scales"], None))
            s_gpu = moe_gpu.grouped_swiglu(d["x"], off1, d["ws1"].unsqueeze(0), d["ws2"].unsqueeze(0))
        torch.cuda.synchronize()
        shared = host(s_gpu)
        assert rel_frobenius(shared[sel], s_ref) <= _tol(cfg)
    y_ref = moe.combine(host(yp), r["row_map"], host(dbg["topk_gates"]), shared)
    e_y = rel_frobenius(host(y), y_ref)
    print(f"[parity-full] {name}: combine rel_frob {e_y:.3e}", flush=True)
    assert e_y <= 4e-3
