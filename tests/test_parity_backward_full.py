"""Backward parity at full size, in the launch configuration `bench.py --backward` times.

The whole backward runs on the GPU; the oracle then recomputes sampled outputs one by one:
* dx of sampled tokens: a token's input gradient depends only on that token's row, its routing
  and the weights, so the oracle backward of the one-token layer gives it exactly;
* dW1 columns f and F + f and dW2 row f of sampled experts, for sampled f: those depend only on
  the same columns of W1 and row of W2, so the oracle's single-expert backward over every row of
  the expert with the sliced weights gives them (dy_perm from the oracle's combine backward);
* the shared expert the same way over all tokens;
* dW_r under softmax without renormalisation: each row sums to zero (the softmax Jacobian's
  rows sum to zero), a property that holds at any size.
Bar: 2e-2 relative Frobenius error on each sampled set (the bf16 bar).
"""

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import backward as obw
from oracle import moe
from tests.checks import rel_frobenius
from tests.gpu_oracle import host, routing_from_logits, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


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
    print(f"[{name}] GPU backward done", flush=True)

    bias = None if d["bias"] is None else host(d["bias"])
    r = routing_from_logits(dbg["logits"], d["bias"], k, cfg.score, cfg.norm, E)
    assert np.array_equal(host(dbg["topk_ids"]), r["ids"])
    x = host(d["x"]).astype(np.float64)
    dyh = host(dy).astype(np.float64)
    wr = host(d["w_router"])
    logits = host(dbg["logits"])
    cache = {}

    def w1_of(e):
        if ("w1", e) not in cache:
            cache[("w1", e)] = weights_of(d["w1"], None, e)
        return cache[("w1", e)]

    def w2_of(e):
        if ("w2", e) not in cache:
            cache[("w2", e)] = weights_of(d["w2"], None, e)
        return cache[("w2", e)]

    sw1 = weights_of(d["ws1"], None, None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], None, None) if cfg.Fs else None
    rng = np.random.default_rng(5)

    # dx of sampled tokens through the oracle backward of each one-token layer
    tokens = sorted(rng.choice(T, 2, replace=False).tolist())
    got, ref = [], []
    for t in tokens:
        fw = moe.forward(x[t:t + 1], wr, w1_of, w2_of, E=E, k=k, score=cfg.score, norm=cfg.norm, bias=bias,
                         shared_w1=sw1, shared_w2=sw2, logits=logits[t:t + 1])
        o = obw.backward(fw, x[t:t + 1], wr, w1_of, w2_of, dyh[t:t + 1], score=cfg.score, norm=cfg.norm,
                         shared_w1=sw1, shared_w2=sw2)
        got.append(host(g["dx"][t]))
        ref.append(o["dx"][0])
    err_dx = rel_frobenius(np.stack(got), np.stack(ref))
    print(f"[{name}] dx on tokens {tokens}: {err_dx:.2e}", flush=True)
    assert err_dx <= TOL

    # dW1 / dW2 slices of the sampled tokens' experts over all of their rows
    dy_perm, _ = obw.combine_backward(dyh, np.zeros((T * k, H)), r["row_map"], r["gates"])
    xp = moe.permute_rows(x, r["src_token"])
    fs = np.sort(rng.choice(F, 3, replace=False))
    cols = np.concatenate([fs, F + fs])
    experts = sorted({int(e) for t in tokens for e in r["ids"][t]})[:4]
    for e in experts:
        a, b = int(r["offsets"][e]), int(r["offsets"][e + 1])
        _, dw1, dw2 = obw.swiglu_expert_backward(xp[a:b], w1_of(e)[:, cols], w2_of(e)[fs, :], dy_perm[a:b])
        e1 = rel_frobenius(host(g["dw1"][e][:, torch.as_tensor(cols, device=DEV)]), dw1)
        e2 = rel_frobenius(host(g["dw2"][e][torch.as_tensor(fs, device=DEV), :]), dw2)
        print(f"[{name}] expert {e} ({b - a} rows), hidden columns {fs.tolist()}: dW1 {e1:.2e} dW2 {e2:.2e}",
              flush=True)
        assert e1 <= TOL and e2 <= TOL
    if cfg.Fs:
        fss = np.sort(rng.choice(cfg.Fs, 3, replace=False))
        scols = np.concatenate([fss, cfg.Fs + fss])
        _, dws1, dws2 = obw.swiglu_expert_backward(x, sw1[:, scols], sw2[fss, :], dyh)
        e1 = rel_frobenius(host(g["dws1"][:, torch.as_tensor(scols, device=DEV)]), dws1)
        e2 = rel_frobenius(host(g["dws2"][torch.as_tensor(fss, device=DEV), :]), dws2)
        print(f"[{name}] shared expert, hidden columns {fss.tolist()}: dWs1 {e1:.2e} dWs2 {e2:.2e}", flush=True)
        assert e1 <= TOL and e2 <= TOL

    if cfg.score == "softmax" and not cfg.norm:
        dwr = host(g["dw_router"]).astype(np.float64)
        rel = np.abs(dwr.sum(axis=1)) / np.linalg.norm(dwr, axis=1)
        print(f"[{name}] dW_r row sums / row norms: max {rel.max():.2e}", flush=True)
        assert rel.max() <= 1e-4
