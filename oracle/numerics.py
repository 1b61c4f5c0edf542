"""Exact widening of stored inputs and rounding to the storage grid (oracle).

Test infrastructure: see the package header for who may import this.
"""
import numpy as np


def widen(a, dtype):
    """Stored array -> float64, exactly.

    ``dtype`` is "bf16" (``a`` holds uint16 bit patterns: a bf16 value is the
    upper half of the float32 with the same sign, exponent and leading 7
    mantissa bits), "f32", or "f64" (pins that feed exact values)."""
    a = np.asarray(a)
    if dtype == "bf16":
        hi = a.astype(np.uint32) * np.uint32(65536)
        return hi.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f64":  # used by pins that feed exact values
        return a.astype(np.float64)
    raise ValueError(dtype)


def round_to_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits.  Writing x = f * 2**e with 0.5 <= |f| < 1,
    the representable neighbours are multiples of 2**(e-8); ``np.rint`` rounds
    half-way cases to the even multiple.  (No overflow or subnormal handling:
    the values met here are far inside bf16's range.)"""
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)


def round_to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype):
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    return np.asarray(x, dtype=np.float64)
