"""FP8 E4M3 KV-cache quantization: the oracle for the fp8 append.

TEST INFRASTRUCTURE ONLY (see the package docstring): not for the product path.

The pages list an fp8 option for the server (TGI architecture page, launcher
options) without its encoding.  The reading taken here: the OCP 8-bit
floating point E4M3 format (1 sign bit, 4 exponent bits with bias 7, 3
mantissa bits; no infinities; S.1111.111 is NaN, so the largest finite
magnitude is 1.75 * 2^8 = 448; exponent field 0 holds subnormals m * 2^-9),
with one fp32 scale per kv head and cache:

    stored byte  = E4M3( x / scale )   x / scale in fp32, then the nearest
                   E4M3 value, ties to the even code (mantissa bit 0 clear),
                   magnitudes beyond 448 saturate to 448
    dequantized  = scale * decode(byte)

Decoding follows the format definition directly; quantization enumerates the
255 finite codes and takes the nearest one, which is obviously correct and
fast enough for tests.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0


def decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 bytes -> exact fp64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    v = s * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _table():
    """Finite non-negative codes 0x00..0x7E and their values, ascending."""
    codes = np.arange(0x7F, dtype=np.int64)
    return codes, decode(codes)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """fp32 values -> E4M3 bytes (uint8) of x / scale, nearest with ties to
    the even code, saturating at +-448.  ``x`` must be finite."""
    q = (np.asarray(x, np.float32) / np.float32(scale)).astype(np.float64)  # fp32 division, exact widening
    mag = np.minimum(np.abs(q), MAX)
    codes, vals = _table()
    hi = np.clip(np.searchsorted(vals, mag, side="left"), 0, len(vals) - 1)  # first value >= mag
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    code = np.where(take_hi, codes[hi], codes[lo])
    code = np.where(mag == vals[hi], codes[hi], code)
    return (code | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """Bytes -> the values attention sees: scale * decode(byte), in fp64."""
    return float(scale) * decode(codes)
