"""FP8 e4m3 ("E4M3FN") encoder and decoder, written from the format's definition.

The pages name FP8 as the precision of the P.V product (juejin page
"MiniMax H3 接入 SageAttention 实测加速", section 一) without giving the format's
details; the definition used here is the OCP 8-bit floating point E4M3 format:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so the largest finite value
is S.1111.110 = 1.75 * 2^8 = 448.

Readings:
* rounding is to nearest, ties to the even mantissa (the IEEE default);
* out-of-range magnitudes saturate to +-448 ("satfinite");
* NaN encodes as 0x7F.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0

__all__ = ["E4M3_MAX", "e4m3_table", "e4m3_decode", "e4m3_encode"]


def _decode_code(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9            # subnormal
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)
# the 127 non-negative finite values, ascending: codes 0x00 .. 0x7E
_POS = _TABLE[:0x7F].copy()


def e4m3_table() -> np.ndarray:
    """All 256 code points decoded to fp64 (NaN at 0x7F and 0xFF)."""
    return _TABLE.copy()


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Round each value (fp32 or fp64) to the nearest e4m3 value, ties to even,
    saturating to +-448; returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
        e = np.maximum(ex - 1, -6)             # binade of a; -6 also covers subnormals
        quantum = np.ldexp(1.0, e - 3)         # spacing of e4m3 values in that binade
        r = np.rint(a / quantum)               # exact scaling, then half-to-even
        val = np.minimum(r * quantum, E4M3_MAX)
        val = np.where(np.isnan(a), 0.0, val)
    code = np.searchsorted(_POS, val).astype(np.uint8)
    assert np.all(_POS[code] == val), "rounded value is not an e4m3 value"
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code
