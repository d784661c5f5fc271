"""Stored number formats, decoded exactly to float64 (oracle; test infrastructure).

bfloat16: the top 16 bits of an IEEE-754 binary32 value.

OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
bits.  Exponent field 0 encodes subnormals (m/8) * 2^-6; fields 1..15 encode
(1 + m/8) * 2^(e-7), except the all-ones pattern S.1111.111 which is NaN.
There is no infinity; the largest finite magnitude is 448.  The pages ask for
a KV cache of about 6 bits per element without naming a scheme ("DeepSeek-V2:
Strong, Economical, Efficient", section 3.2.3, training and inference
efficiency); the fp8
cache with one fp32 scale per token is the 8-bit format of that kind.

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
