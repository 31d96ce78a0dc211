"""Pins of the oracle's MXFP4 codec (oracle/mxfp4.py) against things other than itself.

* E2M1 decode: the 16 values the OCP Microscaling format table lists for E2M1;
* E8M0 decode: torch.float8_e8m0fnu (an independent library) on all 256 bytes;
* E2M1 encode: brute-force nearest-value search over the 16 codes with the tie rule, on every
  midpoint and on random values; identity on every code;
* block scale: linear search for the smallest power of two 2^q with 6 * 2^q >= amax over all
  q in [-127, 127], at exact boundaries, just above and below, and on random magnitudes;
* row quantiser: every element within half a grid step of its value, no scaled element above 6,
  a block's largest magnitude above half the range (the scale is not one power too large);
* packing: element 2i in the low nibble, the byte layout torch's float4_e2m1fn_x2 carries;
* planted mistakes (exponent bias 2, ties to odd, a scale one power too small, swapped nibbles)
  each fail one of these checks.
"""

import math

import numpy as np
import pytest
import torch

from oracle import mxfp4

OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # magnitudes of codes 0..7 in the OCP MX table


def test_decode_matches_the_format_table():
    got = mxfp4.decode_fp4(np.arange(16))
    assert got[:8].tolist() == OCP_E2M1
    assert (got[8:] == -np.array(OCP_E2M1)).all() and np.signbit(got[8])


def test_e8m0_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mxfp4.decode_e8m0(np.arange(256))
    assert np.array_equal(got[:255], ref[:255]) and np.isnan(got[255]) and np.isnan(ref[255])


def _brute_encode(v):
    """Nearest of the 16 code values; on a tie the code with mantissa bit 0; zero as +0."""
    vals = mxfp4.decode_fp4(np.arange(16))
    out = []
    for x in np.asarray(v, dtype=np.float64).ravel():
        x = max(-6.0, min(6.0, x))
        best = None
        for c in range(16):
            d = abs(vals[c] - x)
            if best is None or d < best[0] - 1e-300 or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
                best = (d, c)
        c = best[1]
        out.append(0 if vals[c] == 0 else c)
    return np.array(out, dtype=np.uint8).reshape(np.shape(v))


def test_encode_midpoints_and_random_values_match_brute_force():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    # ties go to the even-mantissa neighbour: 0, 1, 1, 2, 2, 4, 4
    assert mxfp4.decode_fp4(mxfp4.encode_fp4_rne(np.array(mids))).tolist() == [0, 1, 1, 2, 2, 4, 4]
    v = np.concatenate([np.array(mids), -np.array(mids), np.random.default_rng(1).uniform(-6.5, 6.5, 5000),
                        np.nextafter(np.array(mids), 0), np.nextafter(np.array(mids), 7)])
    assert np.array_equal(mxfp4.encode_fp4_rne(v), _brute_encode(v))
    codes = np.arange(16)
    back = mxfp4.encode_fp4_rne(mxfp4.decode_fp4(codes))
    assert back.tolist() == [c if c != 8 else 0 for c in codes]  # -0 encodes as +0


def _brute_scale(amax):
    a = float(np.float32(amax))
    if a == 0.0:
        return 127
    for q in range(-127, 128):
        if 6.0 * math.ldexp(1.0, q) >= a:
            return q + 127
    return 254


def test_block_scale_is_the_smallest_sufficient_power_of_two():
    edges = []
    for q in (-130, -127, -60, -3, -1, 0, 1, 5, 20, 100):
        b = 6.0 * math.ldexp(1.0, q)
        edges += [b, np.nextafter(np.float32(b), np.float32(0)), np.nextafter(np.float32(b), np.float32(np.inf))]
    rng = np.random.default_rng(2)
    amax = np.concatenate([np.array(edges, dtype=np.float32), [0.0, 1e-45, 3.0e38],
                           np.exp(rng.uniform(-80, 80, 3000)).astype(np.float32)]).astype(np.float32)
    got = mxfp4.block_scale_e8m0(amax)
    assert got.tolist() == [_brute_scale(a) for a in amax]


def test_row_quantiser_error_and_range():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    x[3, 32:64] = 0.0  # an all-zero block
    codes, scales = mxfp4.quantise_rows(x)
    s = mxfp4.decode_e8m0(scales)
    assert (s[3, 1] == 1.0)
    deq = mxfp4.dequantise_rows(codes, scales)
    scaled = np.abs(x.reshape(64, 8, 32)) / s[:, :, None]
    assert scaled.max() <= 6.0
    # the grid step around a scaled magnitude m: 0.5 below 2, 1 below 4, 2 above
    step = np.where(scaled < 2, 0.5, np.where(scaled < 4, 1.0, 2.0))
    err = np.abs(deq.reshape(64, 8, 32) - x.reshape(64, 8, 32)) / s[:, :, None]
    assert (err <= step / 2 + 1e-12).all()
    live = x.reshape(64, 8, 32).any(axis=2)
    assert (np.abs(x.reshape(64, 8, 32)).max(axis=2)[live] / s[live] > 3.0).all()


def test_packing_layout():
    codes = np.array([[1, 2, 3, 15, 0, 7]], dtype=np.uint8)
    packed = mxfp4.pack(codes)
    assert packed.tolist() == [[0x21, 0xF3, 0x70]]
    assert np.array_equal(mxfp4.unpack(packed), codes)
    # the same bytes viewed as torch's packed fp4 pairs keep one byte per pair
    t = torch.from_numpy(packed).view(torch.float4_e2m1fn_x2)
    assert t.shape == (1, 3) and t.view(torch.uint8).numpy().tolist() == packed.tolist()


def test_planted_mistakes_are_caught():
    # exponent bias 2 instead of 1: the decoded table is off by a factor of two
    c = np.arange(8)
    wrong = (1.0 + (c & 1) / 2.0) * np.exp2(((c >> 1) & 3) - 2.0)
    wrong = np.where(((c >> 1) & 3) == 0, (c & 1) * 0.5, wrong)
    assert wrong.tolist() != OCP_E2M1
    # ties to the odd code move every midpoint to the other neighbour
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    vals = np.array(OCP_E2M1)
    lo = np.searchsorted(vals, mids) - 1
    odd = np.where(lo % 2 == 1, vals[lo], vals[lo + 1])
    assert odd.tolist() != mxfp4.decode_fp4(mxfp4.encode_fp4_rne(mids)).tolist()
    # a scale one power too small lets scaled values exceed 6
    x = np.full((1, 32), 5.0, dtype=np.float32)
    codes, scales = mxfp4.quantise_rows(x)
    assert scales[0, 0] == 127 and (np.abs(x) / mxfp4.decode_e8m0(scales[0, 0] - 1)).max() > 6
    # swapped nibbles fail the layout check
    c2 = np.array([[1, 2]], dtype=np.uint8)
    assert (c2[:, 1] | (c2[:, 0] << 4)).tolist() != mxfp4.pack(c2)[:, 0].tolist()


def test_mxfp4_layer_mode_quantises_x_and_h():
    """In MXFP4 mode the layer is the plain layer on x quantised per token and h quantised per row
    (1 x 32 blocks), checked against a direct per-token evaluation with the codec; with values
    already on the MXFP4 grid (exactly representable x, and experts whose h lands on the grid)
    the mode changes nothing."""
    from oracle import moe
    rng = np.random.default_rng(4)
    T, H, E, k, F = 12, 64, 4, 2, 32
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((H, E)).astype(np.float32)
    w1 = rng.standard_normal((E, H, 2 * F)) * 0.2
    w2 = rng.standard_normal((E, F, H)) * 0.2
    o = moe.forward(x, wr, lambda e: w1[e], lambda e: w2[e], E=E, k=k, score="softmax", norm=True,
                    mxfp4_mode=True)
    xq = mxfp4.quantised(x)
    assert np.array_equal(o["x_hat"], xq)
    for t in range(T):
        ref = np.zeros(H)
        for j in range(k):
            e = o["ids"][t, j]
            u = xq[t:t + 1] @ w1[e]
            h = mxfp4.quantised(moe.silu(u[:, :F]) * u[:, F:])
            ref += o["gates"][t, j] * (h @ w2[e])[0]
        assert np.allclose(o["y"][t], ref, rtol=1e-12, atol=1e-12)
    # quantising h matters: the unrounded-h layer differs by the 4-bit rounding of h
    plain = moe.forward(xq, wr, lambda e: w1[e], lambda e: w2[e], E=E, k=k, score="softmax", norm=True)
    assert 0.02 < np.linalg.norm(plain["y"] - o["y"]) / np.linalg.norm(plain["y"]) < 0.5


def test_packed_table_decode_equals_the_element_decode():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    scales = rng.integers(100, 150, (7, 2)).astype(np.uint8)
    assert np.array_equal(mxfp4.dequantise_packed(mxfp4.pack(codes), scales), mxfp4.dequantise_rows(codes, scales))
