"""OCP FP8 E4M3 ("e4m3fn") codec and block quantisation -- oracle, test infrastructure only.

The FP8 expert GEMMs of the method (index page of "Scalable Training of
Mixture-of-Experts Models with Megatron Core", abstract; summary page, "Key
claims" [§5] and "Method" second paragraph: selective FP8 on expert GEMMs with
the router kept in higher precision) need an 8-bit float format.  On CDNA4 the
native FP8 is the OCP E4M3 variant without infinities:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals m * 2^-9 (m = 0..7);
* exponent field 1..15 encodes (1 + m/8) * 2^(e-7), except that the single
  pattern S.1111.111 is NaN; so the largest finite magnitude is 1.75 * 2^8 = 448.

Encoding rounds to nearest, ties to the code with an even mantissa LSB, after
the caller has clamped to [-448, 448] (saturating quantisation).

Block quantisation (the reading used throughout, since the pages fix no
scaling recipe; they name FP8 recipes without their scale format): the scale of a
block whose max magnitude is amax > 0 is the smallest power of two 2^q with
448 * 2^q >= amax, q clamped to [-127, 127] (an E8M0 value, the scale format of
MXFP8-style recipes, which the CDNA4 scaled MFMA applies in hardware), else 1;
code = e4m3_rne(clamp(fl32(v / scale), +-448)); the value it stands for is
decode(code) * scale.  Activations use 1x128 blocks along the contraction
dimension, weights 128x128 blocks.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_codes(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 E4M3 codes to float64 from the bit-field definition (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp_field.astype(np.float64) - 7.0)
    subnormal = man * 2.0 ** -9
    mag = np.where(exp_field == 0, subnormal, normal)
    mag = np.where((exp_field == 15) & (man == 7), np.nan, mag)
    return sign * mag


# decode_codes of every byte, so large arrays decode by one table lookup (same values).
_DECODE_TABLE = None


def _decode_table_lookup(codes: np.ndarray) -> np.ndarray:
    global _DECODE_TABLE
    if _DECODE_TABLE is None:
        _DECODE_TABLE = decode_codes(np.arange(256, dtype=np.uint8))
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


# The 127 non-negative finite codes 0x00..0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = decode_codes(_POS_CODES)


def encode_rne(v: np.ndarray) -> np.ndarray:
    """Round float64 values in [-448, 448] to the nearest E4M3 code, ties to even mantissa.

    Nearest-value search over the table of finite codes; the caller clamps first
    (values outside the range are rejected, NaN is rejected).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN cannot be encoded")
    if (np.abs(v) > E4M3_MAX).any():
        raise ValueError("clamp to +-448 before encoding")
    mag = np.abs(v)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")  # first table value >= mag
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_hi = _POS_VALUES[hi] - mag
    d_lo = mag - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((_POS_CODES[lo] & 1) == 0))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi]).astype(np.uint8)
    neg = np.signbit(v) & (code != 0)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def block_scale(amax: np.ndarray) -> np.ndarray:
    """Scale of a block with max magnitude ``amax``: the smallest power of two 2^q with
    448 * 2^q >= amax (q in [-127, 127]), or 1 for an all-zero block; returned as fp32.

    With amax = m * 2^e, m in [0.5, 1) (frexp, exact) and 448 = 0.875 * 2^9, the condition
    reads m * 2^e <= 0.875 * 2^(9 + q), so q = e - 9, plus one when m > 0.875.
    """
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    m, e = np.frexp(a)
    q = np.clip(e - 9 + (m > 0.875), -127, 127)
    s = np.ldexp(1.0, q).astype(np.float32)  # 2^-127 is an exact fp32 (subnormal) value
    return np.where(a > 0, s, np.float32(1.0)).astype(np.float32)


def quantise_block_values(v: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Codes of fp32 values ``v`` under fp32 ``scale`` (broadcast): e4m3_rne(clamp(fl32(v / s)))."""
    q = (np.asarray(v, dtype=np.float32) / np.asarray(scale, dtype=np.float32)).astype(np.float32)
    q = np.clip(q.astype(np.float64), -E4M3_MAX, E4M3_MAX)
    return encode_rne(q)


def quantise_rows_1x128(x: np.ndarray, block: int = 128):
    """Quantise each row of ``x`` [n, K] in 1 x ``block`` blocks along K.

    Returns (codes uint8 [n, K], scales fp32 [n, K/block]).  K must be a multiple of ``block``.
    """
    x = np.asarray(x, dtype=np.float32)
    n, K = x.shape
    if K % block:
        raise ValueError(f"K={K} is not a multiple of {block}")
    xb = x.reshape(n, K // block, block)
    amax = np.abs(xb).max(axis=2)
    s = block_scale(amax)
    codes = quantise_block_values(xb, s[:, :, None]).reshape(n, K)
    return codes, s


def dequantise_rows_1x128(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """float64 values decode(code) * scale of a 1 x ``block`` quantised matrix (exact in fp64)."""
    n, K = codes.shape
    d = _decode_table_lookup(codes).reshape(n, K // block, block)
    return (d * np.asarray(scales, dtype=np.float64)[:, :, None]).reshape(n, K)


def quantise_blocks_128x128(w: np.ndarray, block: int = 128):
    """Quantise a [K, N] matrix in ``block`` x ``block`` tiles. Returns (codes [K, N], scales [K/b, N/b])."""
    w = np.asarray(w, dtype=np.float32)
    K, N = w.shape
    if K % block or N % block:
        raise ValueError(f"shape {w.shape} is not a multiple of {block}")
    wb = w.reshape(K // block, block, N // block, block)
    amax = np.abs(wb).max(axis=(1, 3))
    s = block_scale(amax)
    codes = quantise_block_values(wb, s[:, None, :, None]).reshape(K, N)
    return codes, s


def dequantise_blocks_128x128(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """float64 values decode(code) * scale of a ``block`` x ``block`` quantised [K, N] matrix."""
    K, N = codes.shape
    d = _decode_table_lookup(codes).reshape(K // block, block, N // block, block)
    return (d * np.asarray(scales, dtype=np.float64)[:, None, :, None]).reshape(K, N)
