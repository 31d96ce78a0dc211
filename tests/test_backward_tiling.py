"""CPU model of the backward GEMM's tile bookkeeping (mixture_experts_layer_fp32_amd/csrc/backward.hip).

The index formulas of bwd_gemm_kernel are restated here and checked for coverage: every operand
tile element is loaded and stored by exactly one thread, the LDS swizzle is a permutation of each
row that keeps 16-byte chunks whole, and the XCD-contiguous order of the TN tiles visits every
tile exactly once.  The restated formulas are this model's; the kernel itself is checked by the
GPU parity of the fp32 backward (tests/test_parity_backward.py: the fp32 cases, among them
fp32_multi_group with 9 and 10 m-tiles per weight gradient, run this kernel for every product),
so a formula changed in the kernel but not here fails there, and this model covers the shapes
those cases do not.
"""

import itertools

import pytest

# (BM, BN, BK, bf16): the instantiated tile shapes
SHAPES = [(256, 128, 32, True), (128, 256, 32, True), (128, 128, 16, False)]


def nthreads(BM, BN):
    return BM * BN // 64


def swz(row, k):
    return (((k >> 3) ^ ((row >> 4) & 3)) << 3) | (k & 7)


@pytest.mark.parametrize("BM,BN,BK,bf16", SHAPES)
def test_transposing_loader_covers_each_element_once(BM, BN, BK, bf16):
    NTH = nthreads(BM, BN)
    for cols in (BM, BN):
        CG = cols // 4
        TR = BK * CG // NTH
        assert TR in (2, 4) and (NTH // CG) * TR == BK
        seen = set()
        for tid in range(NTH):
            nb, kq = (tid % CG) * 4, (tid // CG) * TR
            for j, r in itertools.product(range(4), range(TR)):
                seen.add((nb + j, kq + r))
        assert len(seen) == cols * BK == NTH * 4 * TR


@pytest.mark.parametrize("BM,BN,BK,bf16", SHAPES)
def test_chunked_loaders_cover_each_element_once(BM, BN, BK, bf16):
    NTH = nthreads(BM, BN)
    for rows, V in ((BM, 8 if bf16 else 4), (BN, 8 if bf16 else 4)):
        # k-contiguous: chunk c -> row c / (BK / V), k (c % (BK / V)) V
        R = rows * BK // V // NTH
        assert R >= 1 and R * V * NTH == rows * BK
        cells = [(c // (BK // V), c % (BK // V) * V + i) for c in range(R * NTH) for i in range(V)]
        assert len(set(cells)) == len(cells) == rows * BK
        assert all(r < rows and k < BK for r, k in cells)
        # m / n-contiguous: chunk c -> k row c / (rows / V), column (c % (rows / V)) V
        cells = [(c % (rows // V) * V + i, c // (rows // V)) for c in range(R * NTH) for i in range(V)]
        assert len(set(cells)) == len(cells) == rows * BK


def test_swizzle_permutes_each_row_and_keeps_chunks():
    for row in range(256):
        img = [swz(row, k) for k in range(32)]
        assert sorted(img) == list(range(32))
        for c in range(4):  # a 16-byte chunk (8 bf16) stays contiguous and 16-byte aligned
            chunk = img[8 * c:8 * c + 8]
            assert chunk == list(range(chunk[0], chunk[0] + 8)) and chunk[0] % 8 == 0


def test_swizzle_spreads_the_transposed_stores():
    """The A tile's transposed 8-byte stores of one wave (rows 4 apart, same k) fall on at most
    4-way-conflicting banks (64 banks of 4 bytes, 80-byte rows), down from 16-way unswizzled."""
    LD_BYTES = 80

    def worst(swizzled):
        banks = {}
        for lane in range(64):
            row = 4 * lane  # j = 0, kq = 0
            k = swz(row, 0) if swizzled else 0
            b = (row * LD_BYTES + 2 * k) // 4 % 64
            banks[b] = banks.get(b, 0) + 1
        return max(banks.values())
    assert worst(False) == 16
    assert worst(True) <= 4


@pytest.mark.parametrize("tiles", list(range(1, 70)) + [224 * 16, 7168, 1792])
def test_xcd_tile_order_visits_each_tile_once(tiles):
    per = (tiles + 7) // 8
    grid = 8 * per
    got = []
    for w in range(grid):
        L = (w % 8) * per + w // 8
        if L < tiles:
            got.append(L)
    assert sorted(got) == list(range(tiles))
    # each XCD (w % 8) takes one contiguous range of tiles
    for x in range(8):
        mine = [(x * per) + i for i in range(per) if x * per + i < tiles]
        assert mine == [L for w, L in ((w, (w % 8) * per + w // 8) for w in range(grid)) if w % 8 == x and L < tiles]


@pytest.mark.parametrize("rows,S", [(4096, 16), (257, 4), (100, 1), (0, 1), (65536, 32)])
def test_router_row_slices_partition_the_rows(rows, S):
    """TN with one dense group and S slices: slice y takes rows [rows y / S, rows (y + 1) / S)."""
    bounds = [(rows * y // S, rows * (y + 1) // S) for y in range(S)]
    assert bounds[0][0] == 0 and bounds[-1][1] == rows
    assert all(a[1] == b[0] for a, b in zip(bounds, bounds[1:]))


@pytest.mark.parametrize("tiles_m", list(range(1, 20)) + [16, 28, 56])
@pytest.mark.parametrize("tiles_n", [1, 2, 3, 7, 32, 224])
def test_grouped_tn_order_is_a_bijection(tiles_m, tiles_n):
    """Inside an XCD's range, tile L -> groups of 8 m-tiles walked n-major (the last group may be
    narrower): every (m, n) tile exactly once."""
    seen = set()
    for L in range(tiles_m * tiles_n):
        grp, idx = L // (8 * tiles_n), L % (8 * tiles_n)
        gm = min(8, tiles_m - grp * 8)
        m, n = grp * 8 + idx % gm, idx // gm
        assert 0 <= m < tiles_m and 0 <= n < tiles_n
        seen.add((m, n))
    assert len(seen) == tiles_m * tiles_n
