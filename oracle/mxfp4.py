"""MXFP4 (OCP Microscaling) codec -- oracle, test infrastructure only.

The pages name low-precision training in FP8 and NVFP4 ("Scalable Training of Mixture-of-
Experts Models with Megatron Core", index page, abstract; summary page, "Key claims" [§5]);
on CDNA4 the 4-bit counterpart the matrix cores take natively is MXFP4: FP4 E2M1 elements in
blocks of 32 consecutive values along the contraction, each block with one E8M0 (power-of-two)
scale.  The pages fix none of the format's details, so this module states them from the format
definitions (readings, also listed in the design doc):

* E2M1 element: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is the
  subnormal range.  The 8 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.
* Element rounding: to the nearest representable value, ties to the code with mantissa bit 0
  ("even"), after scaling; magnitudes above 6 saturate to 6 (the scale rule below leaves none).
* E8M0 scale: a byte e standing for 2^(e - 127), e = 255 reserved (NaN).
* Block scale (reading, as for the E4M3 path): the smallest power of two 2^q with 6 * 2^q >= the
  block's largest magnitude, q clamped to [-127, 127]; an all-zero block gets 2^0.  No element
  of a block then exceeds the largest E2M1 magnitude after scaling.
* Value of a stored element: decode(code) * 2^(e - 127).
* Packing: two elements per byte, element 2i in the low nibble and 2i + 1 in the high nibble.
* The decision (scale, code) is taken in fp32, the precision the GPU path quantises in: inputs
  are rounded to fp32 first, and x / 2^q is exact in fp32.

Everything here is plain numpy, evaluated element by element from these definitions.
"""

from __future__ import annotations

import numpy as np

FP4_MAX = 6.0
BLOCK = 32
E8M0_BIAS = 127


def decode_fp4(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes (0..15, one per element) -> float64 values, from the bit fields."""
    c = np.asarray(codes).astype(np.int64)
    if ((c < 0) | (c > 15)).any():
        raise ValueError("E2M1 codes are 4-bit")
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    exp_field = (c >> 1) & 3
    man = (c & 1).astype(np.float64)
    normal = (1.0 + man / 2.0) * np.exp2(exp_field.astype(np.float64) - 1.0)
    subnormal = man * 0.5
    return sign * np.where(exp_field == 0, subnormal, normal)


# The 8 non-negative codes in increasing value (decode_fp4 of codes 0..7).
_POS_CODES = np.arange(8, dtype=np.uint8)
_POS_VALUES = decode_fp4(_POS_CODES)


def encode_fp4_rne(v: np.ndarray) -> np.ndarray:
    """Scaled values (|v| <= 6 after saturation) -> E2M1 codes, nearest value, ties to the code
    whose mantissa bit is 0.  -0 and values rounding to 0 encode as +0."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no E2M1 code")
    mag = np.minimum(np.abs(v), FP4_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, mag, side="left"), 0, 7)  # first value >= mag
    lo = np.clip(hi - 1, 0, 7)
    d_lo, d_hi = mag - _POS_VALUES[lo], _POS_VALUES[hi] - mag
    tie = d_lo == d_hi
    pick_lo = (d_lo < d_hi) | (tie & ((_POS_CODES[lo] & 1) == 0))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi]).astype(np.uint8)
    neg = np.signbit(v) & (code != 0)
    return np.where(neg, code | 8, code).astype(np.uint8)


def decode_e8m0(e: np.ndarray) -> np.ndarray:
    """E8M0 bytes -> float64 scales 2^(e - 127); 255 -> NaN."""
    e = np.asarray(e).astype(np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - E8M0_BIAS))


def block_scale_e8m0(amax: np.ndarray) -> np.ndarray:
    """E8M0 byte of the smallest power of two 2^q with 6 * 2^q >= amax (q in [-127, 127]);
    127 (2^0) for an all-zero block.  amax is taken in fp32."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    q = np.ceil(np.log2(np.where(a > 0, a, 1.0) / FP4_MAX))
    # log2 of an fp32 over 6 is exact enough to find the candidate; settle it exactly
    q = np.where(FP4_MAX * np.ldexp(1.0, q.astype(np.int64)) >= a, q, q + 1)
    q = np.where(FP4_MAX * np.ldexp(1.0, (q - 1).astype(np.int64)) >= a, q - 1, q)
    q = np.clip(q, -127, 127)
    return np.where(a > 0, q + E8M0_BIAS, E8M0_BIAS).astype(np.uint8)


def quantise_rows(x: np.ndarray, block: int = BLOCK):
    """x [n, K] -> (codes [n, K] uint8, one E2M1 code per element; scales [n, K / block] E8M0 bytes):
    each row quantised in blocks of `block` consecutive values (fp32 decision)."""
    x = np.asarray(x, dtype=np.float32)
    n, K = x.shape
    if K % block:
        raise ValueError(f"K = {K} is not a multiple of the block {block}")
    xb = x.reshape(n, K // block, block).astype(np.float64)
    e = block_scale_e8m0(np.abs(xb).max(axis=2))
    s = decode_e8m0(e)
    scaled = (xb / s[:, :, None]).astype(np.float32).astype(np.float64)  # exact: s is a power of two
    codes = encode_fp4_rne(np.clip(scaled, -FP4_MAX, FP4_MAX))
    return codes.reshape(n, K), e


def dequantise_rows(codes: np.ndarray, scales: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Inverse of quantise_rows: float64 [n, K]."""
    codes = np.asarray(codes)
    n, K = codes.shape
    d = decode_fp4(codes).reshape(n, K // block, block)
    return (d * decode_e8m0(scales)[:, :, None]).reshape(n, K)


def pack(codes: np.ndarray) -> np.ndarray:
    """[n, K] codes -> [n, K / 2] bytes, element 2i in the low nibble, 2i + 1 in the high one."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    """[n, K / 2] bytes -> [n, K] codes (inverse of pack)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


# decode_fp4 of both nibbles of every byte, so large stored matrices decode by one table lookup
# (the same values as decode_fp4 element by element).
_PAIR_TABLE = None


def dequantise_packed(packed: np.ndarray, scales: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Stored MXFP4 rows ([n, K / 2] packed bytes + [n, K / block] E8M0) -> float64 [n, K]."""
    global _PAIR_TABLE
    if _PAIR_TABLE is None:
        b = np.arange(256, dtype=np.uint8)
        _PAIR_TABLE = np.stack([decode_fp4(b & 0xF), decode_fp4(b >> 4)], axis=1)  # [256, 2]
    p = np.asarray(packed, dtype=np.uint8)
    n, half = p.shape
    d = _PAIR_TABLE[p].reshape(n, half * 2 // block, block)
    return (d * decode_e8m0(scales)[:, :, None]).reshape(n, half * 2)


def quantised(x: np.ndarray) -> np.ndarray:
    """x as the MXFP4 GEMMs see it: quantised per row in 1 x 32 blocks, then decoded (float64)."""
    return dequantise_rows(*quantise_rows(x))
