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


#: the non-negative finite E4M3 values in increasing order, with their codes
_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)  # 0x00..0x7E
_POS_VALUES = E4M3_TABLE[_POS_CODES]


def float_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Encode float32 values to E4M3 codes, rounding to nearest with ties to the even code.

    From the format's definition: the two representable neighbours of ``|x|`` are found among
    the 127 non-negative finite values; the nearer one wins and an exact tie goes to the code
    whose mantissa is even (the lower bit of the code is 0). Magnitudes above 448 are clamped to
    448 (the caller clamps before encoding; nothing here produces NaN for finite input). The
    sign bit is copied, so -0.0 encodes as 0x80. NaN input encodes as 0x7F.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x).astype(np.float64), 448.0)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    v_hi, v_lo = _POS_VALUES[hi], _POS_VALUES[lo]
    d_hi, d_lo = v_hi - a, a - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    pick_hi |= v_hi == a
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)
