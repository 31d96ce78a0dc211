"""Pins of the oracle's Route stage: logits, selection key, top-k, gates."""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import moe


def test_logits_match_explicit_loop():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 24)).astype(np.float32)
    w = (rng.standard_normal((24, 7)) * 0.3).astype(np.float32)
    got = moe.router_logits(x, w)
    assert got.dtype == np.float32
    for t in range(5):
        for e in range(7):
            s = math.fsum(float(x[t, h]) * float(w[h, e]) for h in range(24))  # exact sum, one rounding
            assert abs(float(got[t, e]) - float(np.float32(s))) <= abs(s) * 2 ** -23


def test_one_hot_tokens_return_router_rows():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((16, 6)).astype(np.float32)
    x = np.eye(16, dtype=np.float32)[[3, 0, 15]]
    assert np.array_equal(moe.router_logits(x, w), w[[3, 0, 15]])


def test_topk_all_equal_gives_first_k():
    key = np.zeros((3, 9), dtype=np.float32)
    assert (moe.topk_ids(key, 4) == np.arange(4)).all()


def test_topk_boundary_tie_goes_to_lower_index():
    key = np.array([[0.5, 3.0, 1.0, 2.0, 1.0, 0.0]], dtype=np.float32)
    # 3.0 (e1), 2.0 (e3), then 1.0 at e2 and e4 tie for the last slot: e2 wins
    assert moe.topk_ids(key, 3).tolist() == [[1, 3, 2]]


def test_topk_signed_zero_is_a_tie():
    key = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    assert moe.topk_ids(key, 1).tolist() == [[0]]
    key = np.array([[0.0, -0.0, -1.0]], dtype=np.float32)
    assert moe.topk_ids(key, 2).tolist() == [[0, 1]]


def test_topk_rejects_nonfinite_and_bad_k():
    with pytest.raises(ValueError):
        moe.topk_ids(np.array([[np.nan, 1.0]], dtype=np.float32), 1)
    with pytest.raises(ValueError):
        moe.topk_ids(np.zeros((1, 3), dtype=np.float32), 4)


@settings(max_examples=200, deadline=None)
@given(E=st.integers(1, 10), data=st.data())
def test_topk_matches_exhaustive_subset_search(E, data):
    k = data.draw(st.integers(1, E))
    # small integer keys make ties common
    vals = data.draw(st.lists(st.integers(-3, 3), min_size=E, max_size=E))
    key = (np.array([vals], dtype=np.float32) / 4).astype(np.float32)
    assert moe.topk_ids(key, k)[0].tolist() == moe.brute_force_topk(key[0], k)


def test_permuting_router_columns_permutes_ids():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    w = rng.standard_normal((32, 10)).astype(np.float32)
    perm = rng.permutation(10)
    ids = moe.topk_ids(moe.router_logits(x, w), 3)
    ids_p = moe.topk_ids(moe.router_logits(x, w[:, perm]), 3)
    assert np.array_equal(perm[ids_p], ids)


def test_bias_moves_selection_but_not_gates():
    logits = np.array([[2.0, 1.0, 0.5, 0.0]], dtype=np.float32)
    bias = np.array([-10.0, 0.0, 0.0, 5.0], dtype=np.float32)
    ids = moe.topk_ids(moe.selection_key(logits, bias), 2)
    assert ids.tolist() == [[3, 1]]
    g = moe.gates(logits, ids, moe.SIGMOID, norm=False)
    assert g[0, 0] == 0.5 and g[0, 1] == 1 / (1 + math.exp(-1.0))


def test_selection_key_is_one_fp32_addition():
    # 1 + 2^-24 is not representable in fp32: the key rounds back to 1 (ties to even)
    logits = np.array([[1.0]], dtype=np.float32)
    key = moe.selection_key(logits, np.array([2.0 ** -24], dtype=np.float32))
    assert key.dtype == np.float32 and key[0, 0] == 1.0
    key = moe.selection_key(logits, np.array([3 * 2.0 ** -24], dtype=np.float32))
    assert key[0, 0] == np.float32(1.0 + 2.0 ** -22)


def test_softmax_gates_closed_forms():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((7, 12)).astype(np.float32)
    all_ids = np.tile(np.arange(12), (7, 1))
    p = moe.gates(lg, all_ids, moe.SOFTMAX, norm=False)
    assert np.allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
    # E = 2: p0 = sigmoid(l0 - l1)
    lg2 = np.array([[0.7, -1.3]], dtype=np.float32)
    p2 = moe.gates(lg2, np.array([[0]]), moe.SOFTMAX, norm=False)[0, 0]
    d = float(lg2[0, 0]) - float(lg2[0, 1])
    assert abs(p2 - 1 / (1 + math.exp(-d))) < 1e-15
    # equal logits: 1/E, renormalised: 1/k
    eq = np.zeros((2, 8), dtype=np.float32)
    ids = moe.topk_ids(eq, 3)
    assert np.allclose(moe.gates(eq, ids, moe.SOFTMAX, norm=False), 1 / 8, atol=1e-16)
    assert np.allclose(moe.gates(eq, ids, moe.SOFTMAX, norm=True), 1 / 3, atol=1e-16)


def test_sigmoid_gates_and_normalisation():
    lg = np.array([[0.0, 2.0, -1.0]], dtype=np.float32)
    ids = np.array([[1, 0]])
    g = moe.gates(lg, ids, moe.SIGMOID, norm=False)
    assert g[0, 1] == 0.5 and abs(g[0, 0] - 1 / (1 + math.exp(-2))) < 1e-16
    gn = moe.gates(lg, ids, moe.SIGMOID, norm=True)
    assert abs(gn.sum() - 1.0) < 1e-15
    assert abs(gn[0, 0] / gn[0, 1] - g[0, 0] / g[0, 1]) < 1e-14
