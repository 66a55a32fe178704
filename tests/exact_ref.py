"""Exact rational brute force used to pin the oracle (tests only).

Everything here works on `fractions.Fraction` and on the full list of a format's values, found by
enumerating bit patterns, so it shares no rounding logic with `oracle/`.
"""
from __future__ import annotations

import bisect
import math
import struct
from fractions import Fraction
from functools import lru_cache


def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def _fp16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]


def _e4m3_value(c: int) -> float:
    # OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is subnormal.
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * m / 8.0 * 2.0 ** -6
    return s * (1 + m / 8.0) * 2.0 ** (e - 7)


def _e2m1_value(c: int) -> float:
    s = -1.0 if c & 0x8 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    if e == 0:
        return s * m * 0.5
    return s * (1 + m / 2.0) * 2.0 ** (e - 1)


_DECODERS = {"bf16": (_bf16_value, 16), "fp16": (_fp16_value, 16), "e4m3": (_e4m3_value, 8),
             "e2m1": (_e2m1_value, 4)}


@lru_cache(maxsize=None)
def grid(fmt: str):
    """Sorted (value, bits) of every finite non-negative value of the format."""
    dec, nbits = _DECODERS[fmt]
    sign = 1 << (nbits - 1)
    out = {}
    for c in range(sign):
        v = dec(c)
        if math.isfinite(v):
            out.setdefault(v, c)
    items = sorted(out.items())
    return [Fraction(v) for v, _ in items], [c for _, c in items]


SATURATING = {"e4m3", "e2m1"}


def rne_exact(x: Fraction, fmt: str) -> Fraction:
    """Round the exact rational x to the nearest value of fmt, ties to the even bit pattern.
    bf16/fp16 overflow to infinity per IEEE (returned as None); e4m3/e2m1 saturate."""
    vals, codes = grid(fmt)
    a = abs(x)
    sgn = -1 if x < 0 else 1
    top = vals[-1]
    if a >= top:
        if fmt in SATURATING:
            return sgn * top
        # IEEE: beyond max + half an ulp (ties go to the even side, which is infinity) -> inf
        half = (top - vals[-2]) / 2
        if a >= top + half:
            return None
        return sgn * top
    i = bisect.bisect_right(vals, a)
    lo, hi = vals[i - 1], vals[i]
    if a == lo:
        return sgn * lo
    dlo, dhi = a - lo, hi - a
    if dlo < dhi:
        r = lo
    elif dhi < dlo:
        r = hi
    else:
        r = lo if codes[i - 1] % 2 == 0 else hi
    return sgn * r


def frac(x) -> Fraction:
    return Fraction(float(x))
