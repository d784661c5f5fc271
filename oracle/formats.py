"""Stored number formats, decoded exactly to float64 (oracle; test infrastructure).

bfloat16: the top 16 bits of an IEEE-754 binary32 value.

OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
bits.  Exponent field 0 encodes subnormals (m/8) * 2^-6; fields 1..15 encode
(1 + m/8) * 2^(e-7), except the all-ones pattern S.1111.111 which is NaN.
There is no infinity; the largest finite magnitude is 448.  The pages ask for
a KV cache of about 6 bits per element without naming a scheme ("DeepSeek-V2:
Strong, Economical, Efficient", section 3.2.3, training and inference
efficiency); the fp8 cache with one fp32 scale per token is the 8-bit format
of that kind, and the 6-bit one is below.

OCP microscaling FP6 E2M3 ("MXFP6"): 1 sign bit, 2 exponent bits (bias 1), 3
mantissa bits.  Exponent field 0 encodes subnormals (m/8) * 2^0; fields 1..3
encode (1 + m/8) * 2^(e-1).  No infinity or NaN; the largest magnitude is
7.5.  Blocks of 32 consecutive elements share one E8M0 scale (an 8-bit
biased power of two, 2^(v - 127)): 6 + 8/32 = 6.25 bits per element.

Per-token quantisation rule of the fp8 cache (the quantised code is an integer
decided in float32, the precision the kernel takes it in):
    s    = float32(amax(|row|)) / 448   (float32 division; s = 1 if amax = 0)
    code = the E4M3 value nearest to float32(x / s), ties to even mantissa,
           magnitudes above 448 saturate to 448.
    dequantised value = decode(code) * s
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) exactly to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# The 127 non-negative finite magnitudes, in increasing order: codes 0x00..0x7E.
_POS_VALUES = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 codes (uint8) to float64 through the 256-entry table."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def f32_to_e4m3_rne_sat(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each float32 value (ties to even), saturating."""
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.isnan(v)):
        raise ValueError("NaN has no saturating E4M3 code")
    mag = np.abs(v).astype(np.float64)
    neg = np.signbit(v)
    mag = np.minimum(mag, E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")       # first >= mag
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows_e4m3(rows: np.ndarray):
    """Quantise each row to E4M3 codes with one float32 scale per row.

    rows: float32 [N, D] (the values as the cache-append step sees them).
    Returns (codes uint8 [N, D], scales float32 [N]).
    """
    rows = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(rows), axis=1)
    scale = amax / np.float32(E4M3_MAX)          # float32 division
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    q = rows / scale[:, None]                    # float32 division
    return f32_to_e4m3_rne_sat(q), scale


def dequantize_rows_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 value of each stored element: decode(code) * scale."""
    return e4m3_to_f64(codes) * np.asarray(scales, dtype=np.float64)[:, None]


# ------------------------------------------------------------ MXFP6 E2M3
E2M3_MAX = 7.5
MX_BLOCK = 32                       # elements per shared scale
E2M3_EMAX = 2                       # exponent of the largest normal (7.5 = 1.875 * 2^2)


def _e2m3_value(code: int) -> float:
    sign = -1.0 if code & 0x20 else 1.0
    e = (code >> 3) & 0x3
    m = code & 0x7
    if e == 0:
        return sign * (m / 8.0)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 1)


E2M3_TABLE = np.array([_e2m3_value(c) for c in range(64)], dtype=np.float64)
# The 32 non-negative magnitudes, increasing: codes 0x00..0x1F.
_E2M3_POS = E2M3_TABLE[:32].copy()
assert np.all(np.diff(_E2M3_POS) > 0)


def e2m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode E2M3 codes (6-bit values in uint8) through the 64-entry table."""
    return E2M3_TABLE[np.asarray(codes, dtype=np.uint8) & 0x3F]


def e2m3_nearest_sat(y: np.ndarray) -> np.ndarray:
    """Nearest E2M3 code to each value (ties to the even code), magnitudes
    above 7.5 saturating; the sign bit is the IEEE sign bit of the input."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.isnan(y)):
        raise ValueError("NaN has no E2M3 code")
    mag = np.minimum(np.abs(y), E2M3_MAX)
    hi = np.minimum(np.searchsorted(_E2M3_POS, mag, side="left"), 31)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E2M3_POS[lo]
    d_hi = _E2M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | np.where(np.signbit(y), 0x20, 0)).astype(np.uint8)


def mx_block_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent of a block (the OCP microscaling rule for E2M3):
    floor(log2(amax)) - 2, so that amax / 2^e lies in [4, 8); kept in
    [-126, 127] (an all-zero block takes -126), so 2^e is a normal float32."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E2M3_EMAX
    e = np.where(amax > 0, e, -126)
    return np.clip(e, -126, 127).astype(np.int32)


def quantize_rows_mxfp6(rows: np.ndarray):
    """Quantise each row (length a multiple of 32) to E2M3 codes with one
    E8M0 exponent per block of 32 elements.

    rows: float32 [N, D] (the values as the cache-append step sees them).
    Returns (codes uint8 [N, D] (6-bit values), exps int32 [N, D/32]).
    Dividing by 2^e is exact, so the codes are a property of the float32
    values alone.
    """
    rows = np.asarray(rows, dtype=np.float32).astype(np.float64)
    n, d = rows.shape
    if d % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blocks = rows.reshape(n, d // MX_BLOCK, MX_BLOCK)
    e = mx_block_exponent(np.max(np.abs(blocks), axis=2))
    y = blocks / np.ldexp(1.0, e)[:, :, None]
    return e2m3_nearest_sat(y).reshape(n, d), e


def dequantize_rows_mxfp6(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """float64 value of each stored element: decode(code) * 2^e of its block."""
    codes = np.asarray(codes)
    n, d = codes.shape
    v = e2m3_to_f64(codes).reshape(n, d // MX_BLOCK, MX_BLOCK)
    return (v * np.ldexp(1.0, np.asarray(exps))[:, :, None]).reshape(n, d)


MXFP6_ROW_BYTES = 452               # 576 elements: 432 code bytes, 18 exponents, 2 pad


def pack_rows_mxfp6(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """Byte image of cache rows of 576 elements: 18 blocks of 24 bytes, code
    i of a block at bits 6 i .. 6 i + 5 of the block's 192-bit little-endian
    string; then the 18 exponents as E8M0 bytes (e + 127); then 2 zero bytes.
    """
    codes = np.asarray(codes, dtype=np.uint64)
    n, d = codes.shape
    if d != 576:
        raise ValueError("the packed layout is defined for rows of 576 elements")
    out = np.zeros((n, MXFP6_ROW_BYTES), dtype=np.uint8)
    blocks = codes.reshape(n, 18, 32)
    for k in range(18):
        bits = np.zeros((n, 24 * 8), dtype=np.uint8)
        for i in range(32):
            c = blocks[:, k, i]
            for t in range(6):
                bits[:, 6 * i + t] = (c >> np.uint64(t)) & np.uint64(1)
        for byte in range(24):
            val = np.zeros(n, dtype=np.uint64)
            for t in range(8):
                val |= bits[:, 8 * byte + t].astype(np.uint64) << np.uint64(t)
            out[:, 24 * k + byte] = val.astype(np.uint8)
    out[:, 432:450] = (np.asarray(exps) + 127).astype(np.uint8)
    return out
