"""Exact scalar helpers for the oracle (test infrastructure only).

Every helper here is a plain definition: exponent extraction through
``numpy.frexp`` (exact), bf16 <-> fp32 by bit movement, and round-to-nearest-even
to bf16 from fp64 by rounding the significand to 8 bits. None of them is shared
with the GPU path.
"""
import numpy as np


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> exact float32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_f32(x, dtype):
    """Input tensor as exact float32 values. ``dtype`` is 'f32' or 'bf16' (uint16 bit patterns)."""
    if dtype == "bf16":
        x = bf16_bits_to_f32(x)
    elif dtype == "f32":
        x = np.asarray(x, dtype=np.float32)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the format's domain")
    return x


def floor_log2(a):
    """floor(log2 a) for a > 0 (exact: a = f * 2**e with f in [0.5, 1) gives e - 1)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1


def ceil_log2(a):
    """ceil(log2 a) for a > 0, exact."""
    f, e = np.frexp(np.asarray(a, dtype=np.float64))
    e = e.astype(np.int64)
    return np.where(f == 0.5, e - 1, e)


def significand(a):
    """a / 2**floor(log2 a), in [1, 2), exact for a > 0."""
    f, _ = np.frexp(np.asarray(a, dtype=np.float64))
    return 2.0 * f


def round_f64_to_bf16_bits(v):
    """Round fp64 values to bf16 with round-to-nearest-even, in one rounding. Returns uint16 bits.

    The significand is scaled to 8 integer bits and rounded half-to-even; the
    exact result then fits float32, whose top 16 bits are the bf16 pattern.
    Values below the bf16 normal range are rounded on the subnormal grid
    (quantum 2**-133); the magnitudes here never overflow bf16.
    """
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)  # v = f * 2**e, |f| in [0.5, 1)
    e = np.maximum(e, -125)  # below 2**-126 the quantum stays 2**-133
    q = np.rint(np.ldexp(v, 8 - e))  # round half to even on the 8-bit grid of this binade
    r = np.ldexp(q, e - 8).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def round_f64_to_f32(v):
    """IEEE round-to-nearest-even fp64 -> fp32 (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)
