"""Pins of the oracle's Dispatch stage: counts, offsets, permutation, row copy."""

import numpy as np
import pytest

from oracle import moe
from tests.checks import check_permutation


def _random_ids(T, E, k, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (1, 8, 8), (37, 8, 2), (200, 16, 5), (64, 40, 1)])
def test_permutation_structure(T, E, k):
    ids = _random_ids(T, E, k, T + E)
    cnt = moe.expert_counts(ids, E)
    off = moe.expert_offsets(cnt)
    row_map, src = moe.permutation(ids)
    check_permutation(ids, cnt, off, row_map, src)


def test_permutation_matches_sorted_tuples():
    ids = _random_ids(50, 6, 3, 9)
    row_map, src = moe.permutation(ids)
    tuples = sorted((int(ids[t, j]), t, j) for t in range(50) for j in range(3))
    for p, (_, t, j) in enumerate(tuples):
        assert row_map[t, j] == p and src[p] == t


def test_zero_token_and_all_token_experts():
    T, E = 10, 5
    ids = np.tile(np.array([[4, 1]], dtype=np.int32), (T, 1))  # experts 0, 2, 3 get nothing
    cnt = moe.expert_counts(ids, E)
    assert cnt.tolist() == [0, T, 0, 0, T]
    off = moe.expert_offsets(cnt)
    assert off.tolist() == [0, 0, T, T, T, 2 * T]
    row_map, src = moe.permutation(ids)
    check_permutation(ids, cnt, off, row_map, src)
    assert row_map[:, 1].tolist() == list(range(T)) and row_map[:, 0].tolist() == list(range(T, 2 * T))


def test_permute_rows_is_exact_copy():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((20, 8)).astype(np.float32)
    ids = _random_ids(20, 4, 2, 3)
    row_map, src = moe.permutation(ids)
    xp = moe.permute_rows(x, src)
    for t in range(20):
        for j in range(2):
            assert np.array_equal(xp[row_map[t, j]], x[t])


@pytest.mark.parametrize("mutation", ["swap_rows", "shift_count", "bad_offset", "dup_row", "reverse_expert"])
def test_checker_catches_planted_mistakes(mutation):
    """The permutation checker used by the parity tests must reject a corrupted oracle result."""
    ids = _random_ids(40, 6, 3, 11)
    cnt = moe.expert_counts(ids, 6).copy()
    off = moe.expert_offsets(cnt).copy()
    row_map, src = moe.permutation(ids)
    row_map, src = row_map.copy(), src.copy()
    if mutation == "swap_rows":
        a, b = row_map[0, 0], row_map[5, 1]
        row_map[0, 0], row_map[5, 1] = b, a
    elif mutation == "shift_count":
        cnt[0] += 1
        cnt[1] -= 1
    elif mutation == "bad_offset":
        off[3] += 1
    elif mutation == "dup_row":
        row_map[2, 2] = row_map[3, 0]
    elif mutation == "reverse_expert":
        e = int(np.argmax(cnt))
        seg = slice(off[e], off[e + 1])
        src[seg] = src[seg][::-1].copy()
        for p in range(off[e], off[e + 1]):
            t = src[p]
            j = int(np.where(ids[t] == e)[0][0])
            row_map[t, j] = p
    with pytest.raises(AssertionError):
        check_permutation(ids, cnt, off, row_map, src)
