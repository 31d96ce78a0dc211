"""Checkers shared by the oracle tests and the GPU parity tests (no layer arithmetic here)."""

from __future__ import annotations

import numpy as np


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in float64 (0 when both are empty or ref is all zero and got equals it)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def check_permutation(ids, counts, offsets, row_map, src_token):
    """Structural checks of a dispatch permutation; raises AssertionError on the first violation.

    * counts[e] = #{(t, j): ids[t, j] = e} and they sum to T*k;
    * offsets is the exclusive prefix sum of counts;
    * row_map is a bijection of [0, T*k) and src_token[row_map[t, j]] = t;
    * the rows of expert e are offsets[e]..offsets[e+1]-1, in increasing token order.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    counts = np.asarray(counts, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    row_map = np.asarray(row_map, dtype=np.int64)
    src = np.asarray(src_token, dtype=np.int64)
    E = counts.shape[0]
    assert counts.sum() == T * k, "counts do not sum to T*k"
    assert (np.bincount(ids.ravel(), minlength=E)[:E] == counts).all(), "counts disagree with ids"
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all(), "offsets are not the scan of counts"
    flat = row_map.ravel()
    assert flat.min() >= 0 and flat.max() < T * k, "row_map out of range"
    assert np.unique(flat).size == T * k, "row_map is not a bijection"
    tok = np.repeat(np.arange(T), k)
    assert (src[flat] == tok).all(), "src_token is not the inverse of row_map"
    exp_of_row = np.empty(T * k, dtype=np.int64)
    exp_of_row[flat] = ids.ravel()
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        assert (exp_of_row[a:b] == e).all(), f"rows of expert {e} are not contiguous"
        assert (np.diff(src[a:b]) > 0).all(), f"rows of expert {e} are not in increasing token order"


def max_row_rel(got, ref) -> float:
    """max over rows i of ||got_i - ref_i|| / ||ref_i|| (float64): a bound that one wrong row or tile
    cannot hide behind the whole-tensor norm.  Rows whose reference is all zero must match exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    got = got.reshape(got.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    zero = den == 0.0
    if (num[zero] != 0.0).any():
        return float("inf")
    if zero.all():
        return 0.0
    return float((num[~zero] / den[~zero]).max())
