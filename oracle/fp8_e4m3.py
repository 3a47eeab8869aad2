"""OCP e4m3fn decoding, written from the format's definition (CPU oracle part).

Test infrastructure only: imported by tests, the smoke check and the bench's
CPU-baseline leg, never by the product path.

vllm-metis 0.1.0 ("Status" and "Serve") quantises FP8 with scale = amax / 448;
448 is the largest finite value of the OCP E4M3 "fn" variant (the FNUZ
variant tops out at 240), so that is the encoding decoded here:

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent field 0 -> subnormal, value = (m / 8) * 2**(1 - 7);
* otherwise value = (1 + m / 8) * 2**(e - 7);
* exponent 15 with mantissa 7 (codes 0x7F, 0xFF) is NaN; there are no infinities.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_BIAS = 7
E4M3_MAX = 448.0


def decode_code(code: int) -> float:
    """Value of one e4m3fn code, as a Python float."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


def table() -> np.ndarray:
    """All 256 code values as float64, indexed by code."""
    return np.array([decode_code(c) for c in range(256)], dtype=np.float64)


_TABLE = table()


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to float64 (exact)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# encoding: round to nearest, ties to even, saturating at +-448
# ---------------------------------------------------------------------------
_FINITE_CODES = np.array([c for c in range(0x00, 0x7F)], dtype=np.int64)   # 0 .. 0x7E: +0 .. 448
_FINITE_VALUES = _TABLE[_FINITE_CODES]                                     # increasing


def encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3fn codes, nearest representable value, ties to the
    code with an even mantissa, magnitudes above 448 saturated to 448 (the
    cache-write reading: saturate, never produce NaN from a finite input).

    Works on magnitudes: the positive codes 0x00..0x7E are increasing in value,
    so the two neighbours of |x| are adjacent codes and the tie rule picks the
    even one (mantissa lsb 0).  NaN inputs give the NaN code 0x7F (sign kept).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)   # exact widening
    sign = np.signbit(x)
    a = np.abs(x)
    a = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_FINITE_VALUES, a, side="left")       # first value >= a
    hi = np.minimum(hi, len(_FINITE_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    v_hi, v_lo = _FINITE_VALUES[hi], _FINITE_VALUES[lo]
    d_hi, d_lo = v_hi - a, a - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_FINITE_CODES[hi] % 2 == 0))
    pick_hi |= (v_hi == a)
    code = np.where(pick_hi, _FINITE_CODES[hi], _FINITE_CODES[lo])
    code = np.where(np.isnan(a), 0x7F, code)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)
