"""Number-format helpers of the oracle (exact, definition-based).

Test infrastructure: see the package docstring for who may import this.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact fp64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even) in one rounding step.

    Definition: bf16 has an 8-bit significand and fp32's exponent range, so the
    quantum of a value with binary exponent e is 2^(max(e, -126) - 7).  The value is
    divided by its quantum (exact: a power of two), rounded half-to-even with
    ``np.rint`` and multiplied back.  Zeros keep their sign.  Returns the bf16 *values*
    as fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x * 0.0  # signed zeros stay as they are
    nz = x != 0
    _, e = np.frexp(x[nz])  # x = f * 2^e with f in [0.5, 1)  =>  binary exponent e-1
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    out[nz] = np.rint(x[nz] / q) * q
    big = np.abs(out) >= 2.0 ** 128
    out[big] = np.copysign(np.inf, out[big])
    return out


def bf16_value_to_bits(v: np.ndarray) -> np.ndarray:
    """Exactly-representable bf16 values (fp64) -> uint16 bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def round_f64_to_f32(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest fp32 (IEEE RNE; numpy's cast is correctly rounded)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
