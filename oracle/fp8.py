"""OCP FP8 E4M3 decoding, from the format's bit-field definition (test oracle only).

The pages say only that the KV cache may be held in 8 bits ("serving-paged-attention", section
"실무에서 만지는 지점"). The format is taken to be OCP E4M3: 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 encodes subnormals ``m / 8 * 2**-6``; there are no
infinities; ``S.1111.111`` is NaN, so the largest finite magnitude is ``1.75 * 2**8 = 448``.
"""
from __future__ import annotations

import math

import numpy as np


def _decode_one(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: float64 value of every code 0..255 (NaN for 0x7F and 0xFF)
E4M3_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


def e4m3_to_float(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 E4M3 codes to float64."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
