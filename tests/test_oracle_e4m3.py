"""Pins of the oracle's E4M3 codec against the OCP format and an independent library (torch CPU)."""

import numpy as np
import pytest
import torch

from oracle import e4m3


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3.decode_codes(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.isnan(ours).sum() == 2  # 0x7F and 0xFF only


@pytest.mark.parametrize("code,value", [(0x7E, 448.0), (0x38, 1.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9),
                                        (0x07, 7 * 2.0 ** -9), (0xBC, -1.5), (0x00, 0.0)])
def test_decode_known_values(code, value):
    assert e4m3.decode_codes(np.array([code], dtype=np.uint8))[0] == value


def test_encode_decode_identity_on_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode_rne(e4m3.decode_codes(codes)), codes)


def test_midpoints_round_to_even():
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A: midpoints go to the even mantissa
    assert e4m3.encode_rne(np.array([1.0625]))[0] == 0x38
    assert e4m3.encode_rne(np.array([1.1875]))[0] == 0x3A
    # subnormal midpoint 0.5 * 2^-9 ties to 0, 1.5 * 2^-9 ties to 2 * 2^-9
    assert e4m3.encode_rne(np.array([2.0 ** -10]))[0] == 0x00
    assert e4m3.encode_rne(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    # between 416 (0x7D) and 448 (0x7E): 432 ties to 448 (even 0x7E)
    assert e4m3.encode_rne(np.array([432.0]))[0] == 0x7E


def test_encode_matches_torch_cast_on_random_values():
    rng = np.random.default_rng(5)
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), 20000))
    v = mags * rng.choice([-1.0, 1.0], mags.size)
    v = np.clip(v, -448, 448).astype(np.float32)
    ours = e4m3.encode_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of a value that rounds to zero; the codec returns +0 for both
    ref = np.where((ref & 0x7F) == 0, 0, ref)
    assert np.array_equal(ours, ref)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3.encode_rne(np.array([449.0]))
    with pytest.raises(ValueError):
        e4m3.encode_rne(np.array([np.nan]))


def test_block_quantisation_saturates_and_is_accurate():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    x[2, :128] = 0.0  # an all-zero block gets scale 1 and codes 0
    codes, s = e4m3.quantise_rows_1x128(x)
    assert s.dtype == np.float32 and s.shape == (6, 2)
    assert s[2, 0] == 1.0 and (codes[2, :128] == 0).all()
    xd = e4m3.dequantise_rows_1x128(codes, s)
    # every block's largest magnitude lands in the top binade, (224, 448] -> codes 0x76..0x7E
    for r in range(6):
        for c in range(2):
            blk = x[r, 128 * c:128 * c + 128]
            if np.abs(blk).max() > 0:
                i = np.abs(blk).argmax()
                assert 0x76 <= (codes[r, 128 * c + i] & 0x7F) <= 0x7E
    # normals carry 3 mantissa bits: relative error <= 2^-4; subnormal range: abs error <= 2^-10 * scale
    err = np.abs(xd - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(s, 128, axis=1) * 2.0 ** -10)
    assert (err <= bound * (1 + 1e-12)).all()


def test_weight_block_quantisation_roundtrip():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((256, 384)) * 0.05).astype(np.float32)
    codes, s = e4m3.quantise_blocks_128x128(w)
    assert s.shape == (2, 3)
    wd = e4m3.dequantise_blocks_128x128(codes, s)
    assert np.abs(wd - w).max() <= np.abs(w).max() * 2.0 ** -4
    # a block's scale is the smallest power of two that maps its amax into [-448, 448]
    a = float(np.abs(w[128:, 256:]).max())
    q = min(q for q in range(-130, 131) if 448.0 * 2.0 ** q >= a)
    assert s[1, 2] == np.float32(2.0 ** q)


def test_block_scale_by_search_over_powers_of_two():
    """The scale rule against a direct search: smallest 2^q (q in [-127, 127]) with 448 * 2^q >= amax."""
    rng = np.random.default_rng(5)
    amax = np.concatenate([
        np.float32(448.0) * np.exp2(rng.integers(-40, 40, 200)).astype(np.float32),  # exact 448 * 2^q
        np.nextafter(np.float32(448.0) * np.exp2(rng.integers(-40, 40, 200)).astype(np.float32), np.float32(np.inf)),
        np.exp2(rng.uniform(-140, 120, 3000)).astype(np.float32),
        np.array([1e-45, 1e-40, 2.0 ** -126, 3.4e38, 1.0, 0.875, 0.9, 448.0, 449.0], dtype=np.float32)])
    s = e4m3.block_scale(amax)
    for a, got in zip(amax.astype(np.float64), s):
        cands = [q for q in range(-127, 128) if 448.0 * 2.0 ** q >= a]
        q = min(cands) if cands else 127
        assert got == np.float32(2.0 ** q), (a, got, q)
    assert e4m3.block_scale(np.float32(0.0)) == np.float32(1.0)
    # a block at exactly 448 * 2^q keeps scale 2^q and maps its amax to code 0x7E
    codes, sc = e4m3.quantise_rows_1x128(np.full((1, 128), 448.0 * 2.0 ** -3, dtype=np.float32))
    assert sc[0, 0] == np.float32(2.0 ** -3) and (codes == 0x7E).all()


def test_block_dequantisers_decode_every_code_like_torch():
    """Both dequantisers (table lookup) give torch's E4M3 value times the block scale for all 256 codes."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 128).reshape(128, 256)  # every code in every block
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s_w = np.array([[0.5, 2.0 ** -20]], dtype=np.float32)
    dw = e4m3.dequantise_blocks_128x128(codes, s_w)
    s_r = np.full((128, 2), 4.0, dtype=np.float32)
    s_r[:, 1] = 0.375
    dr = e4m3.dequantise_rows_1x128(codes, s_r)
    for got, scale in ((dw, np.repeat(s_w.astype(np.float64), 128, axis=1)),
                       (dr, np.repeat(s_r.astype(np.float64), 128, axis=1))):
        want = ref * scale
        assert np.array_equal(np.isnan(got), np.isnan(want))
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok])
