"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Per workload (seed 0):
* router logits vs the float64 oracle on all tokens; expert ids, gates, counts, offsets, row_map
  and src_token from the GPU's own logits (bit-exact, all tokens); permuted rows exact (all rows;
  in FP8 the E4M3 codes and 1x128 scales, bit for bit, against the oracle's quantiser);
* expert outputs y_perm on at least 8 sampled rows of EVERY expert that received rows, plus every
  row of 256 sampled tokens, against the oracle's SwiGLU expert on the same (dequantised) rows;
* the layer output y of those 256 tokens against the oracle's own per-token layer: its gates (from
  the GPU's logits), its expert outputs for all k experts of the token, its shared expert;
* combine on all tokens from the GPU's own y_perm; the shared expert alone on the sampled tokens.
Each float comparison has two bars: the relative Frobenius error of the sampled set, and the
largest relative error of any single row, both at the dtype's tolerance, so that one wrong row
or tile cannot hide in the norm of the rest.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import e4m3, moe
from tests.checks import check_permutation, max_row_rel, rel_frobenius
from tests.gpu_oracle import TOL, TOL_GATES, TOL_LOGITS, host, routing_from_logits, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROWS_PER_EXPERT = 8
SAMPLED_TOKENS = 256


def _tol(cfg):
    return TOL["fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype]


def _check(label, got, ref, tol):
    fro, row = rel_frobenius(got, ref), max_row_rel(got, ref)
    print(f"[parity-full] {label}: rel_frob {fro:.3e}, worst row {row:.3e} ({len(ref)} rows)", flush=True)
    assert fro <= tol and row <= tol, label


@pytest.mark.parametrize("name", ["mixtral_8x7b", "qwen3_235b", "deepseek_v3", "deepseek_v3_fp8_zipf"])
def test_full_size_layer(name):
    cfg = moe_inputs.CONFIGS[name]
    T, k, E = cfg.T, cfg.k, cfg.E
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
    r = routing_from_logits(dbg["logits"], d["bias"], k, cfg.score, cfg.norm, E)
    assert np.array_equal(host(dbg["topk_ids"]), r["ids"])
    assert rel_frobenius(host(dbg["topk_gates"]), r["gates"]) <= TOL_GATES
    agree = (moe.topk_ids(moe.selection_key(lg_o, None if d["bias"] is None else host(d["bias"])), k) ==
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
        x_in = e4m3.dequantise_rows_1x128(codes, scales)  # the rows the expert GEMMs see
        del codes, scales
    else:
        assert np.array_equal(host(dbg["x_perm"]), x[r["src_token"]])
        x_in = x
    src = r["src_token"]

    # rows to check: >= 8 of every non-empty expert, and all k rows of the sampled tokens
    cnt, off = r["counts"], r["offsets"]
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(T, SAMPLED_TOKENS, replace=False))
    token_rows = r["row_map"][tokens]  # [S, k]
    picks = {}
    for e in np.nonzero(cnt)[0]:
        a, b = int(off[e]), int(off[e + 1])
        picks[int(e)] = set(rng.choice(np.arange(a, b), min(ROWS_PER_EXPERT, b - a), replace=False).tolist())
    for t_rows, t_ids in zip(token_rows, r["ids"][tokens]):
        for p, e in zip(t_rows, t_ids):
            picks[int(e)].add(int(p))

    def one_expert(e):
        p = np.array(sorted(picks[e]))
        ref = moe.swiglu_expert(x_in[src[p]], weights_of(d["w1"], d["w1_scales"], e),
                                weights_of(d["w2"], d["w2_scales"], e))
        return p, ref

    with ThreadPoolExecutor(8) as ex:  # numpy and the host copies release the interpreter lock
        results = list(ex.map(one_expert, sorted(picks)))
    rows = np.concatenate([p for p, _ in results])
    ref_rows = np.concatenate([ref for _, ref in results])
    yp = dbg["y_perm"]
    got_rows = host(yp[torch.as_tensor(rows, device=DEV, dtype=torch.int64)])
    _check(f"{name} y_perm, {len(picks)} experts", got_rows, ref_rows, _tol(cfg))
    ref_of = dict(zip(rows.tolist(), ref_rows))

    # shared expert on the sampled tokens (alone, through the stage call), then y of those tokens
    shared = s_ref = None
    if cfg.Fs:
        s_ref = moe.swiglu_expert(x_in[tokens], weights_of(d["ws1"], d["ws1_scales"], None),
                                  weights_of(d["ws2"], d["ws2_scales"], None))
        off1 = torch.tensor([0, T], dtype=torch.int32, device=DEV)
        if fp8:  # every token on one expert: permute() is the dense 1x128 quantiser
            q = moe_gpu.permute(d["x"], torch.zeros(T, 1, dtype=torch.int32, device=DEV), 1,
                                perm_dtype=torch.float8_e4m3fn)
            s_gpu = moe_gpu.grouped_swiglu(q["x_perm"], off1, d["ws1"].unsqueeze(0), d["ws2"].unsqueeze(0),
                                           x_perm_scales=q["x_perm_scales"],
                                           w1_scales=d["ws1_scales"].unsqueeze(0),
                                           w2_scales=d["ws2_scales"].unsqueeze(0))
        else:
            s_gpu = moe_gpu.grouped_swiglu(d["x"], off1, d["ws1"].unsqueeze(0), d["ws2"].unsqueeze(0))
        torch.cuda.synchronize()
        shared = host(s_gpu)
        _check(f"{name} shared expert", shared[tokens], s_ref, _tol(cfg))
    yp_local = np.stack([ref_of[int(p)] for p in token_rows.ravel()])
    y_ref = moe.combine(yp_local, np.arange(SAMPLED_TOKENS * k).reshape(SAMPLED_TOKENS, k), r["gates"][tokens],
                        s_ref)
    _check(f"{name} y of {SAMPLED_TOKENS} tokens vs the oracle layer", host(y[torch.as_tensor(tokens, device=DEV)]),
           y_ref, _tol(cfg))
    # combine on all tokens from the GPU's own y_perm (and shared output)
    y_comb = moe.combine(host(yp), r["row_map"], host(dbg["topk_gates"]), shared)
    _check(f"{name} combine of the GPU's y_perm, all tokens", host(y), y_comb, 4e-3)
