"""Number formats of the KV cache, written from the formats' definitions.

"Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
section "Quantization as a way to stretch paged memory further": an FP8 KV
cache halves the BF16 footprint.  The pages do not fix which FP8 variant;
the reading taken here is OCP FP8 E4M3FN (the variant gfx950 implements):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
the all-ones exponent-and-mantissa pattern (S.1111.111) is NaN, largest
finite magnitude 448, subnormals at exponent field 0.

bf16 is the upper half of an IEEE binary32.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (a bf16 is the top 16 bits of a binary32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """Value of one E4M3FN code, straight from the field definition."""
    sign = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)  # subnormal: 0.m * 2^(1-bias)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if sign else mag


_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# positive finite codes 0x00..0x7E in increasing order of value
_POS = _TABLE[:0x7F].copy()


def e4m3_decode_table() -> np.ndarray:
    """All 256 code values as fp64 (NaN for 0x7F and 0xFF)."""
    return _TABLE.copy()


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y) -> np.ndarray:
    """fp32 values -> E4M3FN codes: round to nearest, ties to the even code,
    magnitudes beyond 448 (and +-inf) saturate to +-448, NaN -> 0x7F | sign.

    Done the plain way: locate each magnitude between two adjacent representable
    values and pick the closer one; on an exact tie pick the one whose mantissa
    LSB (= code LSB, since positive codes are consecutive) is 0.
    """
    y32 = np.asarray(y, dtype=np.float32)
    sign = np.signbit(y32)
    a = np.abs(y32.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    hi = np.searchsorted(_POS, a, side="left")  # first code with value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= _POS[0x7E], 0x7E, code)  # saturate
    code = np.where(a == 0.0, 0, code)
    code = np.where(nan, 0x7F, code)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)
