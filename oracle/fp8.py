"""Plain CPU oracle for 8-bit keys and values.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call this module.

[G] 方法详解 (the gptget.net summary of arXiv 2307.02486, method details,
last item) names quantization as an optimisation that combines with the
method; the pages give no format.  Read here as: K and V are stored as FP8
E4M3 codes (the OCP 8-bit floating point format E4M3: sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
m/8 * 2^-6; the all-ones exponent and mantissa pattern is NaN; no infinities;
largest finite value 448) with one float32 scale per (batch, head):

  amax  = max |x| over the head's N rows and D columns (float32),
  inv   = 448 / amax in float32 (1 if amax = 0),
  code  = E4M3 value nearest to float32(x * inv), ties to the even code,
          |x * inv| clamped to 448 first,
  scale = amax / 448 in float32 (1 if amax = 0),

and the attention reads K = decode(code_K) * scale_K, V = decode(code_V) *
scale_V.  Codes are [B, N, H, D] uint8, scales [B, H] float32.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 codes (float64; NaN for the two NaN codes)."""
    vals = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
_POS_CODES = np.array([c for c in range(0x7F)], np.uint8)        # 0x00 .. 0x7E: +0 .. 448
_POS_VALS = _TABLE[:0x7F]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (|x| <= 448), ties to the even code.

    A search over the 127 non-negative finite codes, in ascending value
    order: the candidates are the two codes around |x|; the nearer wins and a
    tie goes to the code whose mantissa is even.  The sign bit is set for
    negative x (negative zero for tiny negative values, as the format keeps it).
    """
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("values must be finite and within +-448")
    hi = np.searchsorted(_POS_VALS, a, side="left")            # first code value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_per_head(x):
    """(codes [B, N, H, D] uint8, scale [B, H] float32) of x [B, N, H, D]."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=(1, 3)).astype(np.float32)          # [B, H]
    nz = amax > 0
    inv = np.where(nz, np.float32(E4M3_MAX) / np.where(nz, amax, np.float32(1)), np.float32(1))
    scale = np.where(nz, amax / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
    y = (x * inv[:, None, :, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(y), scale


def dequantize_per_head(codes, scale) -> np.ndarray:
    """K or V as the attention reads them: decode(code) * scale, float64."""
    return _TABLE[np.asarray(codes, np.uint8)] * np.asarray(scale, np.float64)[:, None, :, None]
