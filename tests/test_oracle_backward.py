"""Pins of the oracle's backward (oracle/backward.py) against finite differences and closed forms.

The forward used here is the oracle's own stage functions composed with float64 router
logits (no fp32 rounding), so the loss L = <dy, y> is smooth in every parameter as long
as the top-k selection does not change; each check asserts that it does not.  Central
differences in float64 then fix every gradient to ~1e-9 relative: a dropped term, a wrong
sign or a transposed operand in the backward fails them.
"""

import numpy as np
import pytest

from oracle import backward as bw
from oracle import moe


def make_params(rng, T, H, E, k, F, Fs, bias):
    p = {
        "x": rng.standard_normal((T, H)),
        "w_router": rng.standard_normal((H, E)) / np.sqrt(H),
        "w1": rng.standard_normal((E, H, 2 * F)) / np.sqrt(H),
        "w2": rng.standard_normal((E, F, H)) / np.sqrt(F),
    }
    if Fs:
        p["ws1"] = rng.standard_normal((H, 2 * Fs)) / np.sqrt(H)
        p["ws2"] = rng.standard_normal((Fs, H)) / np.sqrt(Fs)
    p["bias"] = rng.standard_normal(E) * 0.5 if bias else None
    return p


def forward64(p, k, score, norm, ids=None):
    """The layer in float64 through the oracle's stage functions; returns the forward dict."""
    E = p["w_router"].shape[1]
    lg = p["x"] @ p["w_router"]
    key = lg if p["bias"] is None else lg + p["bias"]
    sel = moe.topk_ids(key, k)
    if ids is not None:
        assert np.array_equal(sel, ids), "perturbation changed the expert selection"
    fw = {"logits": lg, "ids": sel, "gates": moe.gates(lg, sel, score, norm)}
    fw["offsets"] = moe.expert_offsets(moe.expert_counts(sel, E))
    fw["row_map"], src = moe.permutation(sel)
    fw["x_perm"] = moe.permute_rows(p["x"], src)
    fw["y_perm"] = moe.grouped_experts(fw["x_perm"], fw["offsets"], lambda e: p["w1"][e], lambda e: p["w2"][e])
    shared = moe.swiglu_expert(p["x"], p["ws1"], p["ws2"]) if "ws1" in p else None
    fw["y"] = moe.combine(fw["y_perm"], fw["row_map"], fw["gates"], shared)
    return fw


def run_backward(p, fw, dy, score, norm):
    return bw.backward(fw, p["x"], p["w_router"], lambda e: p["w1"][e], lambda e: p["w2"][e], dy,
                       score=score, norm=norm, shared_w1=p.get("ws1"), shared_w2=p.get("ws2"))


GRADS = {"x": "dx", "w_router": "dw_router", "w1": "dw1", "w2": "dw2", "ws1": "dws1", "ws2": "dws2"}


def check_directional(p, k, score, norm, rng, eps=1e-5, directions=3):
    fw = forward64(p, k, score, norm)
    dy = rng.standard_normal(fw["y"].shape)
    g = run_backward(p, fw, dy, score, norm)
    for name, gname in GRADS.items():
        if name not in p:
            assert g[gname] is None
            continue
        for _ in range(directions):
            v = rng.standard_normal(p[name].shape)
            lo, hi = dict(p), dict(p)
            lo[name] = p[name] - eps * v
            hi[name] = p[name] + eps * v
            fd = (np.sum(dy * forward64(hi, k, score, norm, fw["ids"])["y"])
                  - np.sum(dy * forward64(lo, k, score, norm, fw["ids"])["y"])) / (2 * eps)
            an = np.sum(g[gname] * v)
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("score,norm", [("softmax", False), ("softmax", True), ("sigmoid", True), ("sigmoid", False)])
def test_directional_derivatives(score, norm):
    rng = np.random.default_rng(11)
    p = make_params(rng, T=9, H=6, E=5, k=2, F=4, Fs=0, bias=False)
    check_directional(p, 2, score, norm, rng)


def test_directional_derivatives_shared_bias_empty_experts():
    """Shared expert, a selection bias (no gradient) and experts that receive no rows (zero dW)."""
    rng = np.random.default_rng(12)
    p = make_params(rng, T=3, H=6, E=8, k=2, F=4, Fs=3, bias=True)
    fw = forward64(p, 2, "sigmoid", True)
    empty = np.flatnonzero(np.diff(fw["offsets"]) == 0)
    assert len(empty) >= 2
    g = run_backward(p, fw, rng.standard_normal(fw["y"].shape), "sigmoid", True)
    assert not g["dw1"][empty].any() and not g["dw2"][empty].any()
    check_directional(p, 2, "sigmoid", True, rng)


def test_single_expert_is_a_dense_mlp():
    """E = k = 1 with softmax: the gate is identically 1, so no gradient reaches the router."""
    rng = np.random.default_rng(13)
    p = make_params(rng, T=7, H=5, E=1, k=1, F=3, Fs=0, bias=False)
    fw = forward64(p, 1, "softmax", False)
    g = run_backward(p, fw, rng.standard_normal(fw["y"].shape), "softmax", False)
    assert np.max(np.abs(g["dlogits"])) < 1e-15 and np.max(np.abs(g["dw_router"])) < 1e-14
    check_directional(p, 1, "softmax", False, rng)


@pytest.mark.parametrize("score,norm", [("softmax", False), ("sigmoid", True), ("softmax", True)])
def test_identical_experts_give_no_router_gradient(score, norm):
    """With k = E the gates sum to 1 (softmax over all E, or any gates renormalised), so if every
    expert is the same function the output does not depend on the logits: dL/dlogits = 0 while
    each gate's own gradient is not zero."""
    rng = np.random.default_rng(14)
    p = make_params(rng, T=6, H=5, E=4, k=4, F=3, Fs=0, bias=False)
    p["w1"][:] = p["w1"][0]
    p["w2"][:] = p["w2"][0]
    fw = forward64(p, 4, score, norm)
    g = run_backward(p, fw, rng.standard_normal(fw["y"].shape), score, norm)
    assert np.max(np.abs(g["dgate"])) > 0.1
    assert np.max(np.abs(g["dlogits"])) < 1e-13
    assert np.max(np.abs(g["dw_router"])) < 1e-12


def test_sigmoid_without_norm_router_gradient_is_local():
    """sigmoid gates without renormalisation: dL/dlogit is zero on unselected experts and
    dgate * s (1 - s) on selected ones (the logistic function's derivative)."""
    rng = np.random.default_rng(15)
    T, E, k = 5, 6, 2
    lg = rng.standard_normal((T, E))
    ids = moe.topk_ids(lg, k)
    dg = rng.standard_normal((T, k))
    dl = bw.gates_backward(lg, ids, dg, "sigmoid", False)
    s = 1 / (1 + np.exp(-np.take_along_axis(lg, ids, axis=1)))
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids, True, axis=1)
    assert not dl[~mask].any()
    assert np.allclose(np.take_along_axis(dl, ids, axis=1), dg * s * (1 - s), rtol=1e-14, atol=0)


def test_silu_grad_matches_central_difference():
    z = np.linspace(-30, 30, 601)
    eps = 1e-6
    fd = (moe.silu(z + eps) - moe.silu(z - eps)) / (2 * eps)
    assert np.allclose(bw.silu_grad(z), fd, rtol=1e-7, atol=1e-9)


@pytest.mark.parametrize("mutation", ["silu_grad_drops_term", "softmax_drops_mean", "norm_drops_mean",
                                      "dgate_uses_wrong_slot"])
def test_pins_catch_planted_mistakes(monkeypatch, mutation):
    """Plausible mistakes planted in the oracle's backward fail the directional checks."""
    rng = np.random.default_rng(16)
    score, norm = ("softmax", True) if mutation != "softmax_drops_mean" else ("softmax", False)
    if mutation == "silu_grad_drops_term":
        monkeypatch.setattr(bw, "silu_grad", bw.logistic)
    elif mutation in ("softmax_drops_mean", "norm_drops_mean"):
        real = np.sum

        def no_mean(a, axis=None, keepdims=False, **kw):
            out = real(a, axis=axis, keepdims=keepdims, **kw)
            return out * 0 if keepdims and axis == 1 else out
        monkeypatch.setattr(bw.np, "sum", no_mean)
    else:
        real_cb = bw.combine_backward

        def shifted(dy, y_perm, row_map, gate):
            dyp, dg = real_cb(dy, y_perm, row_map, gate)
            return dyp, dg[:, ::-1].copy()
        monkeypatch.setattr(bw, "combine_backward", shifted)
    p = make_params(rng, T=9, H=6, E=5, k=2, F=4, Fs=0, bias=False)
    with pytest.raises(AssertionError):
        check_directional(p, 2, score, norm, rng)
