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
