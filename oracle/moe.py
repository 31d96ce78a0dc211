"""The dropless MoE layer forward as its plain definition -- oracle, test infrastructure only.

Source of the method: "Scalable Training of Mixture-of-Experts Models with
Megatron Core", summary page, section "Method", first paragraph.  The layer is
four stages:

* Route    -- a learned linear projection of every token (optionally in FP32),
              softmax or sigmoid scores, and top-k expert selection;
* Dispatch -- permute the (token, slot) pairs so that rows routed to the same
              expert are contiguous, which is what a dense grouped GEMM needs;
* Compute  -- every local expert (a SwiGLU MLP here) applied to its contiguous
              rows, all experts in one grouped GEMM;
* Combine  -- un-permute and sum each token's k expert outputs weighted by its
              gates; an optional shared expert sees every token.

Permutation and grouping only reorder work, so the oracle is the definition
evaluated stage by stage in float64, plus an independent pure-Python per-token
loop (``brute_force_layer``) for tiny inputs.  Points the pages leave open are
fixed by the readings listed in each docstring (the plainest reading the rest of
the pages support):

R1 scores are taken over all E experts, then the k selected entries are kept;
   gates are renormalised over the k only when ``norm`` is set.
R2 selection ranks fp32 keys: the fp32 router logit, plus (only when a routing
   bias is given) that bias, added in one fp32 addition.  Gates always come from
   the unbiased logit.
R3 ties break to the lower expert index, and slots are ordered by key
   descending (equal keys: index ascending); -0.0 equals +0.0.
R4 inside an expert the rows follow increasing token index.
R5 the 2F columns of the first expert matrix are [gate | up]: h = SiLU(u[:, :F]) * u[:, F:],
   SiLU(z) = z / (1 + e^-z), no biases.
R6 the shared expert has gate 1 and is added after the routed sum.
R7 in FP8 mode the oracle runs on the dequantised operands (x quantised per
   token in 1x128 blocks, weights given as 128x128-block codes + scales) and
   keeps the SwiGLU activation h unrounded.
R8 in MXFP4 mode (oracle/mxfp4.py) both operands of both expert GEMMs are MXFP4:
   x quantised per token in 1x32 blocks, weights given as 32-element-block codes
   + E8M0 scales (dequantised by the caller), and the SwiGLU activation h
   quantised per row in 1x32 blocks before the second GEMM (the operand the
   second GEMM takes is MXFP4 too); the quantisation decision is taken in fp32.
R9 with the gate folded into the experts (``gate_in_expert``, memory-efficient permutation),
   h of each permuted row is multiplied by that row's gate before it is rounded, and
   combine adds the k rows with weight 1: in exact arithmetic the same layer; where h is
   quantised (R8) the quantiser sees g h.

No stage here is blocked, fused or reordered beyond what its definition states;
numpy matmul / argsort / bincount are the only library steps.
"""

from __future__ import annotations

from itertools import combinations
import math

import numpy as np

from . import e4m3, mxfp4

SOFTMAX = "softmax"
SIGMOID = "sigmoid"


# --------------------------------------------------------------------------- Route
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """Router projection: logits[t, e] = fl32(sum_h x[t, h] * W_r[h, e]).

    The summary page ("Method", first paragraph) describes the router as a learned
    linear projection that may be evaluated in FP32; the fp64 sum is rounded once
    to fp32.  ``x`` [T, H] is taken at its stored value (fp32, or bf16 widened
    exactly); ``w_router`` is [H, E] fp32.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_router, dtype=np.float64)
    return (x64 @ w64).astype(np.float32)


def selection_key(logits: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """Key ranked by top-k: the fp32 logit, plus the routing bias in one fp32 add (reading R2)."""
    logits = np.asarray(logits, dtype=np.float32)
    if bias is None:
        return logits
    return (logits + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)


def topk_ids(key: np.ndarray, k: int) -> np.ndarray:
    """Top-k selection (summary page, "Method"): the k largest keys of every token.

    A stable sort of -key gives slots ordered by key descending with equal keys in
    increasing expert index, so ties break to the lower index (reading R3).
    Returns int32 [T, k].
    """
    key = np.asarray(key, dtype=np.float32)
    if not np.isfinite(key).all():
        raise ValueError("router keys must be finite")
    E = key.shape[1]
    if not 1 <= k <= E:
        raise ValueError(f"k={k} must be in [1, E={E}]")
    neg = -key.astype(np.float64) + 0.0  # +0.0 folds -0.0 into +0.0
    order = np.argsort(neg, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates(logits: np.ndarray, ids: np.ndarray, score: str, norm: bool) -> np.ndarray:
    """Gate weights of the selected experts, float64 [T, k] (summary page, "Method": softmax or sigmoid).

    softmax: p = exp(l - max l) / sum_e exp(l - max l) over all E, then the selected
    entries (reading R1).  sigmoid: 1 / (1 + exp(-l)) of the selected logits.
    With ``norm`` the k gates of a token are divided by their sum.
    """
    l64 = np.asarray(logits, dtype=np.float64)
    ids = np.asarray(ids)
    if score == SOFTMAX:
        m = l64.max(axis=1, keepdims=True)
        p = np.exp(l64 - m)
        p = p / p.sum(axis=1, keepdims=True)
        g = np.take_along_axis(p, ids, axis=1)
    elif score == SIGMOID:
        g = 1.0 / (1.0 + np.exp(-np.take_along_axis(l64, ids, axis=1)))
    else:
        raise ValueError(f"unknown score function {score!r}")
    if norm:
        g = g / g.sum(axis=1, keepdims=True)
    return g


# ------------------------------------------------------------------------ Dispatch
def expert_counts(ids: np.ndarray, E: int) -> np.ndarray:
    """counts[e] = number of (token, slot) pairs routed to expert e; int64 [E]."""
    return np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.int64)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum: offsets[0] = 0, offsets[e + 1] = offsets[e] + counts[e]; int64 [E + 1]."""
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def permutation(ids: np.ndarray):
    """Dispatch permutation making each expert's rows contiguous (summary page, "Method").

    The (t, j) pairs, enumerated token-major, are stably sorted by expert id; the
    pair at sorted position p gets row_map[t, j] = p and src_token[p] = t.  A token
    selects an expert at most once, so inside one expert rows follow increasing
    token index (reading R4).  Returns (row_map int64 [T, k], src_token int64 [T*k]).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.ravel().astype(np.int64)
    order = np.argsort(flat, kind="stable")  # order[p] = t*k + j
    row_map = np.empty(T * k, dtype=np.int64)
    row_map[order] = np.arange(T * k, dtype=np.int64)
    src_token = order // k
    return row_map.reshape(T, k), src_token


def permute_rows(x: np.ndarray, src_token: np.ndarray) -> np.ndarray:
    """x_perm[p] = x[src_token[p]] -- an exact row copy."""
    return np.asarray(x)[np.asarray(src_token)]


# ------------------------------------------------------------------------- Compute
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z), float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_expert(rows: np.ndarray, w1: np.ndarray, w2: np.ndarray, h_quant=None, row_scale=None) -> np.ndarray:
    """One SwiGLU expert on a block of rows, float64 (reading R5).

    u = rows @ W1 with W1 [H, 2F]; h = SiLU(u[:, :F]) * u[:, F:]; out = h @ W2 with W2 [F, H].
    h is not rounded, except by ``h_quant`` when given (MXFP4 mode, reading R8: the second GEMM's
    operand is h quantised per row); ``row_scale`` [n] multiplies h row by row first (R9).
    """
    r64 = np.asarray(rows, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    F = w2.shape[0]
    if w1.shape[1] != 2 * F:
        raise ValueError(f"W1 has {w1.shape[1]} columns, expected 2F = {2 * F}")
    u = r64 @ w1
    h = silu(u[:, :F]) * u[:, F:]
    if row_scale is not None:
        h = h * np.asarray(row_scale, dtype=np.float64)[:, None]
    if h_quant is not None:
        h = h_quant(h)
    return h @ w2


def swiglu_hidden(rows: np.ndarray, w1: np.ndarray) -> np.ndarray:
    """The SwiGLU activation h = SiLU(u[:, :F]) * u[:, F:] of one expert, float64 (for diagnostics)."""
    u = np.asarray(rows, dtype=np.float64) @ np.asarray(w1, dtype=np.float64)
    F = u.shape[1] // 2
    return silu(u[:, :F]) * u[:, F:]


def grouped_experts(x_perm: np.ndarray, offsets: np.ndarray, w1_of, w2_of, h_quant=None,
                    row_scale=None) -> np.ndarray:
    """Apply expert e to rows offsets[e]:offsets[e+1] of ``x_perm`` for every e (the grouped GEMM).

    ``w1_of(e)`` / ``w2_of(e)`` return expert e's [H, 2F] / [F, H] weights (so a caller
    can widen one expert at a time); experts with no rows are skipped; ``h_quant`` and
    ``row_scale`` ([R], one per permuted row) as for swiglu_expert.  Returns float64 [R, H].
    """
    x_perm = np.asarray(x_perm)
    R = x_perm.shape[0]
    y = None
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        out = swiglu_expert(x_perm[a:b], w1_of(e), w2_of(e), h_quant,
                            None if row_scale is None else np.asarray(row_scale)[a:b])
        if y is None:
            y = np.zeros((R, out.shape[1]), dtype=np.float64)
        y[a:b] = out
    if y is None:
        y = np.zeros((R, 0), dtype=np.float64)
    return y


# ------------------------------------------------------------------------- Combine
def combine(y_perm: np.ndarray, row_map: np.ndarray, gate: np.ndarray, shared: np.ndarray | None = None):
    """y[t] = sum_j gate[t, j] * y_perm[row_map[t, j]] (+ shared[t], gate 1; reading R6), float64."""
    y_perm = np.asarray(y_perm, dtype=np.float64)
    row_map = np.asarray(row_map)
    g = np.asarray(gate, dtype=np.float64)
    T, k = row_map.shape
    y = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        y += g[:, j:j + 1] * y_perm[row_map[:, j]]
    if shared is not None:
        y += np.asarray(shared, dtype=np.float64)
    return y


# ---------------------------------------------------------------------- the layer
def quantised_input(x: np.ndarray) -> np.ndarray:
    """x as the FP8 expert GEMMs see it: per-token 1x128 E4M3 quantisation, dequantised (reading R7)."""
    codes, scales = e4m3.quantise_rows_1x128(np.asarray(x, dtype=np.float32))
    return e4m3.dequantise_rows_1x128(codes, scales)


def forward(x, w_router, w1_of, w2_of, *, E, k, score, norm, bias=None, shared_w1=None,
            shared_w2=None, fp8=False, mxfp4_mode=False, logits=None, gate_in_expert=False):
    """The whole layer, stage by stage; returns a dict of every intermediate.

    ``x`` [T, H] float array; ``w_router`` [H, E]; ``w1_of(e)``/``w2_of(e)`` give expert
    weights (dequantised values in FP8 / MXFP4 mode); ``shared_w1``/``shared_w2`` the shared
    expert or None.  ``fp8``: reading R7; ``mxfp4_mode``: reading R8; ``gate_in_expert``: R9
    (then ``y_perm`` holds the gate-weighted rows).  If ``logits`` is given (fp32 [T, E]) routing is driven from those
    logits instead of recomputing them -- this is how the GPU's own logits are checked
    bit-exactly for ids / counts / offsets / permutation.
    """
    x = np.asarray(x)
    out = {}
    out["logits_oracle"] = router_logits(x, w_router)
    lg = out["logits_oracle"] if logits is None else np.asarray(logits, dtype=np.float32)
    out["logits"] = lg
    out["key"] = selection_key(lg, bias)
    out["ids"] = topk_ids(out["key"], k)
    out["gates"] = gates(lg, out["ids"], score, norm)
    out["counts"] = expert_counts(out["ids"], E)
    out["offsets"] = expert_offsets(out["counts"])
    out["row_map"], out["src_token"] = permutation(out["ids"])
    if fp8 and mxfp4_mode:
        raise ValueError("one low-precision mode at a time")
    h_quant = mxfp4.quantised if mxfp4_mode else None
    if fp8:
        xq = quantised_input(x)
    elif mxfp4_mode:
        xq = mxfp4.quantised(x)
    else:
        xq = np.asarray(x, dtype=np.float64)
    out["x_hat"] = xq
    out["x_perm"] = permute_rows(xq, out["src_token"])
    g_perm = None
    if gate_in_expert:  # each permuted row's gate: g_perm[row_map[t, j]] = gates[t, j]
        g_perm = np.empty(out["row_map"].size, dtype=np.float64)
        g_perm[out["row_map"].ravel()] = out["gates"].ravel()
    out["y_perm"] = grouped_experts(out["x_perm"], out["offsets"], w1_of, w2_of, h_quant, g_perm)
    shared = None
    if shared_w1 is not None:
        shared = swiglu_expert(xq, shared_w1, shared_w2, h_quant)
    out["shared"] = shared
    weights = np.ones_like(out["gates"]) if gate_in_expert else out["gates"]
    out["y"] = combine(out["y_perm"], out["row_map"], weights, shared)
    return out


# --------------------------------------------------------------- brute force (tiny)
def brute_force_layer(x, w_router, w1, w2, *, k, score, norm, bias=None, shared_w1=None,
                      shared_w2=None):
    """The layer token by token in pure Python floats: no sort, no permutation, no numpy matmul.

    For tiny inputs only.  Per token: logits by explicit sums (rounded to fp32 via
    numpy.float32 on the scalar), keys, the k winners by repeated scans for the
    largest key (lower index wins a tie), gates, and sum_j g_j * SwiGLU_{e_j}(x_t)
    (+ shared expert).  ``w1`` [E, H, 2F] and ``w2`` [E, F, H] as nested sequences or arrays.
    Returns (y [T][H] list of lists, ids [T][k]).
    """
    x = [[float(v) for v in row] for row in np.asarray(x, dtype=np.float64)]
    wr = np.asarray(w_router, dtype=np.float64)
    T, H = len(x), len(x[0])
    E = wr.shape[1]
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)

    def expert_out(w1e, w2e, xt):
        F = len(w2e)
        hidden = []
        for f in range(F):
            g = sum(xt[i] * float(w1e[i][f]) for i in range(H))
            u = sum(xt[i] * float(w1e[i][F + f]) for i in range(H))
            hidden.append(g / (1.0 + math.exp(-g)) * u)
        return [sum(hidden[f] * float(w2e[f][o]) for f in range(F)) for o in range(H)]

    ys, all_ids = [], []
    for t in range(T):
        lg = [float(np.float32(sum(x[t][i] * float(wr[i][e]) for i in range(H)))) for e in range(E)]
        if bias is None:
            key = lg[:]
        else:
            key = [float(np.float32(np.float32(lg[e]) + np.float32(bias[e]))) for e in range(E)]
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or key[e] > key[best]:
                    best = e
            chosen.append(best)
        if score == SOFTMAX:
            m = max(lg)
            z = sum(math.exp(v - m) for v in lg)
            g = [math.exp(lg[e] - m) / z for e in chosen]
        else:
            g = [1.0 / (1.0 + math.exp(-lg[e])) for e in chosen]
        if norm:
            s = sum(g)
            g = [v / s for v in g]
        yt = [0.0] * H
        for j, e in enumerate(chosen):
            o = expert_out(w1[e], w2[e], x[t])
            yt = [yt[i] + g[j] * o[i] for i in range(H)]
        if shared_w1 is not None:
            o = expert_out(np.asarray(shared_w1, dtype=np.float64), np.asarray(shared_w2, dtype=np.float64), x[t])
            yt = [yt[i] + o[i] for i in range(H)]
        ys.append(yt)
        all_ids.append(chosen)
    return ys, all_ids


def brute_force_topk(key_row, k):
    """Top-k of one token by exhaustive search over all C(E, k) expert subsets.

    The answer is the subset whose members, listed by (key descending, index
    ascending), form the lexicographically smallest sequence of (-key, index) pairs.
    For E <= 10 only.
    """
    key_row = [float(v) + 0.0 for v in key_row]
    best = None
    for subset in combinations(range(len(key_row)), k):
        seq = sorted((-key_row[e], e) for e in subset)
        if best is None or seq < best:
            best = seq
    return [e for _, e in best]
