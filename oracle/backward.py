"""Gradients of the dropless MoE layer forward -- oracle, test infrastructure only.

The pages measure the layer in training ("Scalable Training of Mixture-of-Experts
Models with Megatron Core", abstract; summary page, "Method", second paragraph:
fine-grained activation recomputation), so the layer also runs backward.  Given
the upstream gradient dy = dL/dy of the layer output, this module returns
dL/dx, dL/dW_r, dL/dW1[e], dL/dW2[e] and the shared expert's weight gradients.
They are the chain rule applied to the forward's stages (oracle.moe), evaluated
in float64, stage by stage in reverse:

* Combine  y_t = sum_j g_tj yp[row_map(t, j)] + s_t:
             dyp[row_map(t, j)] = g_tj dy_t,  dg_tj = <dy_t, yp[row_map(t, j)]>,  ds_t = dy_t.
* Compute  per expert e on its rows: u = xp W1, a = u[:, :F], b = u[:, F:],
           h = SiLU(a) b, yp = h W2:
             dh = dyp W2^T,  dW2 = h^T dyp,
             da = dh b SiLU'(a) with SiLU'(z) = s(z) (1 + z (1 - s(z))), s the logistic function,
             db = dh SiLU(a),  dxp = [da | db] W1^T,  dW1 = xp^T [da | db].
* Dispatch dx_t = sum_j dxp[row_map(t, j)]   (the permutation is a row copy).
* Route    gates g from the selected scores s_j (softmax over all E taken at the
           selected experts, or the logistic function of the selected logit),
           divided by their sum S when ``norm``:
             norm:  ds_j = (dg_j - sum_i dg_i g_i) / S;  else ds_j = dg_j;
             softmax: dl_e = p_e (ds~_e - sum_j ds_j p_{id_j}), ds~_e = ds_j where e = id_j, else 0;
             sigmoid: dl_{id_j} = ds_j s_j (1 - s_j), 0 for unselected experts;
           then dx_t += dl_t W_r^T and dW_r = x^T dl.
           Top-k selection and the selection bias are piecewise constant: no gradient
           flows through them.
* Shared expert (gate 1): the Compute rule on all T rows with dyp = dy.

The routing (ids, gates, permutation) is taken from the forward's result dict, so
the same bits drive both directions.  FP8 expert GEMMs are not differentiated here.
"""

from __future__ import annotations

import numpy as np

from .moe import SIGMOID, SOFTMAX, silu


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def logistic(z: np.ndarray) -> np.ndarray:
    """s(z) = 1 / (1 + e^-z), float64."""
    return 1.0 / (1.0 + np.exp(-_f64(z)))


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z s(z)] = s(z) + z s(z) (1 - s(z)) = s(z) (1 + z (1 - s(z)))."""
    s = logistic(z)
    return s * (1.0 + _f64(z) * (1.0 - s))


def combine_backward(dy: np.ndarray, y_perm: np.ndarray, row_map: np.ndarray, gate: np.ndarray):
    """Backward of y_t = sum_j g_tj yp[row_map(t, j)]: returns (dy_perm [R, H], dgate [T, k])."""
    dy = _f64(dy)
    y_perm = _f64(y_perm)
    row_map = np.asarray(row_map)
    g = _f64(gate)
    T, k = row_map.shape
    dy_perm = np.zeros_like(y_perm)
    dgate = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        dy_perm[row_map[:, j]] = g[:, j:j + 1] * dy
        dgate[:, j] = np.sum(dy * y_perm[row_map[:, j]], axis=1)
    return dy_perm, dgate


def swiglu_expert_backward(rows: np.ndarray, w1: np.ndarray, w2: np.ndarray, dout: np.ndarray):
    """Backward of out = (SiLU(u[:, :F]) * u[:, F:]) W2, u = rows W1 (one expert, float64).

    Returns (d_rows [n, H], dW1 [H, 2F], dW2 [F, H]).
    """
    r64, w1, w2, dout = _f64(rows), _f64(w1), _f64(w2), _f64(dout)
    F = w2.shape[0]
    u = r64 @ w1
    a, b = u[:, :F], u[:, F:]
    h = silu(a) * b
    dh = dout @ w2.T
    dw2 = h.T @ dout
    du = np.concatenate([dh * b * silu_grad(a), dh * silu(a)], axis=1)
    return du @ w1.T, r64.T @ du, dw2


def grouped_experts_backward(x_perm: np.ndarray, offsets: np.ndarray, w1_of, w2_of, dy_perm: np.ndarray):
    """Per-expert SwiGLU backward over the contiguous row blocks of ``x_perm``.

    Returns (dx_perm [R, H], dW1 [E, H, 2F], dW2 [E, F, H]); experts without rows get
    zero weight gradients.
    """
    x_perm = _f64(x_perm)
    E = len(offsets) - 1
    w1_0, w2_0 = _f64(w1_of(0)), _f64(w2_of(0))
    dx_perm = np.zeros_like(x_perm)
    dw1 = np.zeros((E,) + w1_0.shape, dtype=np.float64)
    dw2 = np.zeros((E,) + w2_0.shape, dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        dx_perm[a:b], dw1[e], dw2[e] = swiglu_expert_backward(x_perm[a:b], w1_of(e), w2_of(e), dy_perm[a:b])
    return dx_perm, dw1, dw2


def unpermute_backward(dx_perm: np.ndarray, row_map: np.ndarray) -> np.ndarray:
    """Backward of x_perm[row_map(t, j)] = x_t: dx_t = sum_j dx_perm[row_map(t, j)]."""
    dx_perm = _f64(dx_perm)
    row_map = np.asarray(row_map)
    dx = np.zeros((row_map.shape[0], dx_perm.shape[1]), dtype=np.float64)
    for j in range(row_map.shape[1]):
        dx += dx_perm[row_map[:, j]]
    return dx


def gates_backward(logits: np.ndarray, ids: np.ndarray, dgate: np.ndarray, score: str, norm: bool) -> np.ndarray:
    """dL/dlogits [T, E] from dL/dgates [T, k] (the gate definition of oracle.moe.gates)."""
    l64 = _f64(logits)
    ids = np.asarray(ids)
    dg = _f64(dgate)
    T, E = l64.shape
    if score == SOFTMAX:
        m = l64.max(axis=1, keepdims=True)
        p = np.exp(l64 - m)
        p = p / p.sum(axis=1, keepdims=True)
        s = np.take_along_axis(p, ids, axis=1)
    elif score == SIGMOID:
        s = logistic(np.take_along_axis(l64, ids, axis=1))
    else:
        raise ValueError(f"unknown score function {score!r}")
    if norm:
        S = s.sum(axis=1, keepdims=True)
        g = s / S
        ds = (dg - np.sum(dg * g, axis=1, keepdims=True)) / S
    else:
        ds = dg
    dl = np.zeros((T, E), dtype=np.float64)
    if score == SOFTMAX:
        np.put_along_axis(dl, ids, ds, axis=1)  # ds~: ids are distinct within a token
        dl = p * (dl - np.sum(ds * s, axis=1, keepdims=True))
    else:
        np.put_along_axis(dl, ids, ds * s * (1.0 - s), axis=1)
    return dl


def backward(fw: dict, x, w_router, w1_of, w2_of, dy, *, score, norm, shared_w1=None, shared_w2=None):
    """Gradients of L = <dy, y> for the layer whose forward result dict is ``fw``.

    ``fw`` is oracle.moe.forward's output for these inputs (its ``logits`` drive the
    gates, so passing the GPU's logits there differentiates the same routing).
    Returns a dict with dx [T, H], dw_router [H, E], dw1 [E, H, 2F], dw2 [E, F, H],
    dws1 / dws2 (or None) and the intermediates dy_perm, dgate, dlogits, dx_perm.
    """
    x64 = _f64(x)
    out = {}
    dy_perm, dgate = combine_backward(dy, fw["y_perm"], fw["row_map"], fw["gates"])
    dx_perm, out["dw1"], out["dw2"] = grouped_experts_backward(fw["x_perm"], fw["offsets"], w1_of, w2_of, dy_perm)
    dx = unpermute_backward(dx_perm, fw["row_map"])
    dl = gates_backward(fw["logits"], fw["ids"], dgate, score, norm)
    dx += dl @ _f64(w_router).T
    out["dw_router"] = x64.T @ dl
    out["dws1"] = out["dws2"] = None
    if shared_w1 is not None:
        dxs, out["dws1"], out["dws2"] = swiglu_expert_backward(x64, shared_w1, shared_w2, dy)
        dx += dxs
    out.update(dx=dx, dy_perm=dy_perm, dgate=dgate, dlogits=dl, dx_perm=dx_perm)
    return out
