"""IEEE-754 binary16 helpers for the oracle (test infrastructure only).

Written from the binary16 definition (1 sign bit, 5 exponent bits with bias
15, 10 fraction bits; exponent 0 = subnormal, 31 = Inf/NaN), not from any
GPU conversion routine.  Pinned in tests against numpy's float16 over all
65536 bit patterns and over round-to-nearest-even tie cases.
"""
from __future__ import annotations

import math

import numpy as np


def decode_bits(h: int) -> float:
    """Exact float value of a binary16 bit pattern."""
    sign = -1.0 if (h >> 15) & 1 else 1.0
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 0x1F:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -24)            # f * 2^-14 * 2^-10
    return sign * math.ldexp(1024 + f, e - 25)      # (1 + f/1024) * 2^(e-15)


_DECODE_TABLE = None


def decode_array(bits: np.ndarray) -> np.ndarray:
    """Vectorised exact decode of a uint16 (or float16 viewed as uint16)
    array to float64, through a 65536-entry table built by decode_bits."""
    global _DECODE_TABLE
    if _DECODE_TABLE is None:
        _DECODE_TABLE = np.array([decode_bits(h) for h in range(1 << 16)],
                                 dtype=np.float64)
    if bits.dtype == np.float16:
        bits = bits.view(np.uint16)
    return _DECODE_TABLE[bits.astype(np.int64)]


def encode_rne(x: float) -> int:
    """Round a float to the nearest binary16, ties to even; overflow -> Inf."""
    if math.isnan(x):
        return 0x7E00
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a == 0.0:
        return sign
    if math.isinf(a):
        return sign | 0x7C00
    e = math.floor(math.log2(a))
    # guard against log2 rounding at binade edges
    if math.ldexp(1.0, e) > a:
        e -= 1
    elif math.ldexp(1.0, e + 1) <= a:
        e += 1
    e = max(e, -14)                       # subnormal binade shares 2^-14 spacing
    quantum = math.ldexp(1.0, e - 10)     # spacing of representable values
    q = a / quantum                       # exact: power-of-two scaling
    n = math.floor(q)
    rem = q - n
    if rem > 0.5 or (rem == 0.5 and n % 2 == 1):
        n += 1
    value = n * quantum
    if value >= 65536.0:                  # rounded past the largest finite
        return sign | 0x7C00
    # re-derive bits from the rounded value
    if value < math.ldexp(1.0, -14):      # subnormal (or rounds into normal)
        return sign | int(round(value / math.ldexp(1.0, -24)))
    eb = math.floor(math.log2(value))
    if math.ldexp(1.0, eb) > value:
        eb -= 1
    elif math.ldexp(1.0, eb + 1) <= value:
        eb += 1
    frac = int(value / math.ldexp(1.0, eb - 10)) - 1024
    return sign | ((eb + 15) << 10) | frac


def ulp16(x: float) -> float:
    """Spacing of binary16 values at |x|: 2^(max(floor(log2|x|), -14) - 10);
    ulp16(0) = 2^-24."""
    a = abs(float(x))
    if a == 0.0:
        return math.ldexp(1.0, -24)
    e = math.floor(math.log2(a))
    if math.ldexp(1.0, e) > a:
        e -= 1
    elif math.ldexp(1.0, e + 1) <= a:
        e += 1
    return math.ldexp(1.0, max(e, -14) - 10)


def ulp16_array(x: np.ndarray) -> np.ndarray:
    """Vectorised ulp16 via frexp (exact)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(a)                   # a = mant * 2^ex, mant in [0.5, 1)
    e = np.maximum(ex - 1, -14)
    out = np.ldexp(1.0, e - 10)
    return np.where(a == 0.0, math.ldexp(1.0, -24), out)


def rne16_array(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest binary16 value (ties to even), as float64.

    Library step: numpy's float64 -> float16 conversion, which rounds once
    to nearest-even; tests pin it against ``encode_rne``."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
