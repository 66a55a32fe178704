"""Comparison rules of the parity tests (test infrastructure).

Values: the finalize sums in float32 before its one rounding, and float32 cannot always land on
the same side of a bf16/fp16 rounding midpoint as the exact sum. The admissible window is the
rigorous float32 error bound of any evaluation order: with n = 2K + 3 rounded operations on the
path of one element and u = 2^-24,
    |fl32(S*) - S*| <= gamma_n * (|RSF| * sum |w x| + |shared|),  gamma_n = n u / (1 - n u).
The window is padded by 2^-20 of itself to also cover the FP64 oracle's own error (< 2^-46).
An element passes when its rounded value lies between RNE_T(S* - E) and RNE_T(S* + E).

Indices, route selection and quantized codes are compared bit for bit.
"""
from __future__ import annotations

import numpy as np

import oracle as O

U32 = 2.0 ** -24


def fp32_error_bound(mag: np.ndarray, K: int) -> np.ndarray:
    n = 2 * K + 3
    gamma = n * U32 / (1 - n * U32)
    return gamma * mag * (1 + 2.0 ** -20)


def admissible_bounds(S_star, mag, K, act_dtype):
    fmt = O.FORMATS[act_dtype]
    E = fp32_error_bound(mag, K)
    return O.round_to_format(S_star - E, fmt), O.round_to_format(S_star + E, fmt)


def ordered(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers ordered like their values (+0 and -0 both -> 0)."""
    b = bits.astype(np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Number of representable 16-bit values between two patterns (bf16 or fp16)."""
    return np.abs(ordered(np.asarray(a_bits)) - ordered(np.asarray(b_bits)))


def values_to_bits(v, act_dtype):
    return O.encode_bits(v, O.FORMATS[act_dtype])


def bits_to_values(bits, act_dtype):
    return O.decode_bits(bits, O.FORMATS[act_dtype])


def spacing(x, act_dtype) -> np.ndarray:
    """Distance from |x| to the next larger value of the format (its ulp)."""
    fmt = O.FORMATS[act_dtype]
    _, E = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.ldexp(1.0, np.maximum(E - 1, fmt.emin) - fmt.frac_bits)


def outside(values, lo, hi) -> np.ndarray:
    """Mask of elements outside [lo, hi] (NaN counts as outside)."""
    v = np.asarray(values, dtype=np.float64)
    return ~((v >= lo) & (v <= hi))
