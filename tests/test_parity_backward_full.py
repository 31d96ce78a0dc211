"""Backward parity at full size, in the launch configuration `bench.py --backward` times.

The whole backward runs on the GPU; the oracle then recomputes sampled outputs:
* dx of 32 sampled tokens.  A token's input gradient depends only on its own row, its routing and
  the weights, so the oracle backward restricted to the sampled tokens gives it exactly: their
  routing (from the GPU's logits) permuted by the oracle, the combine backward, every expert's
  SwiGLU backward on its rows, the unpermute backward, the gate backward, the router and the
  shared expert -- the oracle's own stage functions, in the order oracle.backward composes them;
* dW1 columns f and F + f and dW2 row f of every expert those tokens use, for 3 sampled hidden
  units f, over all of the expert's rows: they depend only on the same columns of W1 and row of
  W2, so the oracle's single-expert backward with the sliced weights gives them (dy_perm from the
  oracle's combine backward); the shared expert the same way over all tokens;
* dW_r over all tokens: the gate gradients from the oracle's combine backward driven by the GPU's
  own y_perm (as the forward's combine check is), then the oracle's gate backward and x^T dlogits;
  under softmax without renormalisation, also the zero row sums of the softmax Jacobian.
Bars: 2e-2 (the bf16 bar) on the relative Frobenius error of each sampled set and on the worst
single row of it (a token's dx, a hidden unit's dW1 column or dW2 row, a row of dW_r).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import backward as obw
from oracle import moe
from tests.checks import max_row_rel, rel_frobenius
from tests.gpu_oracle import host, routing_from_logits, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2
SAMPLED_TOKENS = 32


def _check(label, got, ref):
    fro, row = rel_frobenius(got, ref), max_row_rel(got, ref)
    print(f"[bwd-full] {label}: rel_frob {fro:.3e}, worst row {row:.3e}", flush=True)
    assert fro <= TOL and row <= TOL, label


@pytest.mark.parametrize("name", ["mixtral_8x7b", "deepseek_v3"])
def test_full_size_backward(name):
    cfg = moe_inputs.CONFIGS[name]
    T, H, E, k, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    _, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    dy = moe_inputs.make_upstream_grad(cfg, seed=0, device=DEV)
    g = moe_gpu.backward(d["x"], dy, layer, dbg)
    torch.cuda.synchronize()
    print(f"[bwd-full] {name}: GPU backward done", flush=True)

    r = routing_from_logits(dbg["logits"], d["bias"], k, cfg.score, cfg.norm, E)
    assert np.array_equal(host(dbg["topk_ids"]), r["ids"])
    x = host(d["x"]).astype(np.float64)
    dyh = host(dy).astype(np.float64)
    wr = host(d["w_router"])
    logits = host(dbg["logits"])
    sw1 = weights_of(d["ws1"], None, None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], None, None) if cfg.Fs else None
    rng = np.random.default_rng(5)

    # the sampled tokens as a layer of their own: the oracle's permutation of their routing
    tokens = np.sort(rng.choice(T, SAMPLED_TOKENS, replace=False))
    ids_s, gates_s = r["ids"][tokens], r["gates"][tokens]
    off_s = moe.expert_offsets(moe.expert_counts(ids_s, E))
    row_map_s, src_s = moe.permutation(ids_s)
    xp_s = moe.permute_rows(x[tokens], src_s)
    dy_perm_s, _ = obw.combine_backward(dyh[tokens], np.zeros((SAMPLED_TOKENS * k, H)), row_map_s, gates_s)
    # all rows of every expert: dy_perm from the combine backward; permuted rows from x
    dy_perm, _ = obw.combine_backward(dyh, np.zeros((T * k, H)), r["row_map"], r["gates"])
    fs = np.sort(rng.choice(F, 3, replace=False))
    cols = np.concatenate([fs, F + fs])
    experts = sorted({int(e) for e in ids_s.ravel()})

    def one_expert(e):
        w1, w2 = weights_of(d["w1"], None, e), weights_of(d["w2"], None, e)
        a_s, b_s = int(off_s[e]), int(off_s[e + 1])
        yp = moe.swiglu_expert(xp_s[a_s:b_s], w1, w2)
        dxp, _, _ = obw.swiglu_expert_backward(xp_s[a_s:b_s], w1, w2, dy_perm_s[a_s:b_s])
        a, b = int(r["offsets"][e]), int(r["offsets"][e + 1])
        _, dw1, dw2 = obw.swiglu_expert_backward(x[r["src_token"][a:b]], w1[:, cols], w2[fs, :], dy_perm[a:b])
        return e, (a_s, b_s), yp, dxp, dw1, dw2

    with ThreadPoolExecutor(8) as ex:  # numpy and the host copies release the interpreter lock
        results = list(ex.map(one_expert, experts))
    del dy_perm
    yp_s = np.zeros((SAMPLED_TOKENS * k, H))
    dxp_s = np.zeros((SAMPLED_TOKENS * k, H))
    got1, ref1, got2, ref2 = [], [], [], []
    cols_t = torch.as_tensor(cols, device=DEV)
    fs_t = torch.as_tensor(fs, device=DEV)
    for e, (a_s, b_s), yp, dxp, dw1, dw2 in results:
        yp_s[a_s:b_s], dxp_s[a_s:b_s] = yp, dxp
        got1.append(host(g["dw1"][e][:, cols_t]).T)  # one row per hidden column, over H
        ref1.append(dw1.T)
        got2.append(host(g["dw2"][e][fs_t, :]))
        ref2.append(dw2)
    _check(f"{name} dW1 columns {cols.tolist()} of {len(experts)} experts", np.concatenate(got1), np.concatenate(ref1))
    _check(f"{name} dW2 rows {fs.tolist()} of {len(experts)} experts", np.concatenate(got2), np.concatenate(ref2))

    # dx of the sampled tokens, composed as oracle.backward composes the stages
    _, dgate_s = obw.combine_backward(dyh[tokens], yp_s, row_map_s, gates_s)
    dx_s = obw.unpermute_backward(dxp_s, row_map_s)
    dl_s = obw.gates_backward(logits[tokens], ids_s, dgate_s, cfg.score, cfg.norm)
    dx_s += dl_s @ wr.astype(np.float64).T
    if cfg.Fs:
        dxs, dws1, dws2 = obw.swiglu_expert_backward(x[tokens], sw1, sw2, dyh[tokens])
        dx_s += dxs
        fss = np.sort(rng.choice(cfg.Fs, 3, replace=False))
        scols = np.concatenate([fss, cfg.Fs + fss])
        _, dws1, dws2 = obw.swiglu_expert_backward(x, sw1[:, scols], sw2[fss, :], dyh)
        _check(f"{name} shared dWs1 columns", host(g["dws1"][:, torch.as_tensor(scols, device=DEV)]).T, dws1.T)
        _check(f"{name} shared dWs2 rows", host(g["dws2"][torch.as_tensor(fss, device=DEV), :]), dws2)
    _check(f"{name} dx of {SAMPLED_TOKENS} tokens", host(g["dx"][torch.as_tensor(tokens, device=DEV)]), dx_s)

    # dW_r over all tokens, the gate gradients driven by the GPU's own y_perm
    dwr_ref = np.zeros((H, E))
    chunk = 512
    for t0 in range(0, T, chunk):
        c = np.arange(t0, min(T, t0 + chunk))
        rows = torch.as_tensor(r["row_map"][c].ravel(), device=DEV, dtype=torch.int64)
        yp_c = host(dbg["y_perm"][rows]).astype(np.float64)
        _, dgate_c = obw.combine_backward(dyh[c], yp_c, np.arange(len(c) * k).reshape(len(c), k), r["gates"][c])
        dl_c = obw.gates_backward(logits[c], r["ids"][c], dgate_c, cfg.score, cfg.norm)
        dwr_ref += x[c].T @ dl_c
    dwr = host(g["dw_router"]).astype(np.float64)
    _check(f"{name} dW_r (all tokens)", dwr, dwr_ref)
    if cfg.score == "softmax" and not cfg.norm:
        rel = np.abs(dwr.sum(axis=1)) / np.linalg.norm(dwr, axis=1)
        print(f"[bwd-full] {name} dW_r row sums / row norms: max {rel.max():.2e}", flush=True)
        assert rel.max() <= 1e-4
