"""f32 -> bf16 conversions: stochastic rounding (SR) and round-to-nearest-even.

bf16 values are held as their 16-bit patterns (numpy uint16), f32 values as
float32 or as their 32-bit patterns (uint32); numpy has no bf16 type.

SR, as the FlyDSL page "Add stochastic rounding and philox RNG helpers"
(Primitives section) describes it: the 16 low bits of the f32 pattern, which
bf16 drops, receive 16 random bits by integer addition, and the sum is then
truncated to its high half. A carry out of the low half happens for exactly
L of the 65,536 possible random values, L being the dropped bits, so the
probability of moving up one bf16 step equals the fractional distance to it
(the page's Tests section: exact unbiasedness over the whole 16-bit range).

Reading taken where the page is wrong: the page says Inf and NaN need no
special case. That holds for +-Inf and for the default quiet NaN, but a NaN
whose payload sits only in the low 16 bits would truncate to Inf, and a NaN
with all-ones low bits would carry into the sign bit or wrap to zero. The
plain reading of "NaN passes through" is that a NaN stays a NaN, so a NaN
input maps to its high half with the quiet bit set, (u >> 16) | 0x0040,
whatever the random bits. Finite values are never saturated: a value near
FLT_MAX may round up to Inf, as round-to-nearest does too.

RN (the comparison mode; the FlyDSL page's Consumer section keeps "rn" as
the default rounding): round to nearest, ties to even, with the same NaN rule.
"""

import struct

import numpy as np

_EXP = 0x7F800000
_MANT = 0x007FFFFF
_QUIET16 = 0x0040


def f32_bits(x):
    """float32 array -> uint32 bit patterns (copy-free view when possible)."""
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def bits_f32(u):
    """uint32 bit patterns -> float32 array."""
    return np.ascontiguousarray(u, dtype=np.uint32).view(np.float32)


def bf16_to_f32(h):
    """bf16 patterns (uint16) -> float32, exactly (the pattern is the high half)."""
    return bits_f32(np.asarray(h, dtype=np.uint32) << np.uint32(16))


def _is_nan_bits(u):
    return ((u & np.uint32(_EXP)) == np.uint32(_EXP)) & ((u & np.uint32(_MANT)) != 0)


def sr_bf16(u, r16):
    """Stochastic rounding, vectorized ("Add stochastic rounding and philox RNG
    helpers", Primitives: add the random bits to the 16 dropped bits, keep the
    high half; a NaN keeps its high half with the quiet bit set).

    ``u``: uint32 f32 patterns; ``r16``: random values in [0, 65536)
    (any unsigned integer array, broadcast against ``u``).
    Returns uint16 bf16 patterns.
    """
    u = np.asarray(u, dtype=np.uint32).astype(np.uint64)
    r = np.asarray(r16).astype(np.uint64)
    if np.any(r > 0xFFFF):
        raise ValueError("random values must be 16-bit")
    summed = ((u + r) & np.uint64(0xFFFFFFFF)) >> np.uint64(16)
    nan_out = (u >> np.uint64(16)) | np.uint64(_QUIET16)
    out = np.where(_is_nan_bits(u.astype(np.uint32)), nan_out, summed)
    return out.astype(np.uint16)


def sr_bf16_scalar(u, r16):
    """Stochastic rounding of one f32 pattern ``u`` with one 16-bit ``r16``
    (the same rule as :func:`sr_bf16`, one value at a time)."""
    u = int(u) & 0xFFFFFFFF
    r16 = int(r16)
    if not 0 <= r16 <= 0xFFFF:
        raise ValueError("random value must be 16-bit")
    if (u & _EXP) == _EXP and (u & _MANT):
        return (u >> 16) | _QUIET16
    return ((u + r16) & 0xFFFFFFFF) >> 16


def rn_bf16(u):
    """Round to nearest, ties to even, vectorized: uint32 patterns -> uint16
    (the comparison mode, "rn", of the FlyDSL pull request's Consumer section)."""
    u = np.asarray(u, dtype=np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    nan_out = (u >> np.uint64(16)) | np.uint64(_QUIET16)
    out = np.where(_is_nan_bits(u.astype(np.uint32)), nan_out, rounded)
    return out.astype(np.uint16)


def rn_bf16_scalar(u):
    """Round to nearest even of one f32 pattern, decided by comparing the
    dropped half with one half of a bf16 step (not by the add trick above)."""
    u = int(u) & 0xFFFFFFFF
    if (u & _EXP) == _EXP and (u & _MANT):
        return (u >> 16) | _QUIET16
    hi, lo = u >> 16, u & 0xFFFF
    if lo > 0x8000 or (lo == 0x8000 and (hi & 1)):
        hi += 1  # magnitude step up; 0x7F7F -> 0x7F80 becomes Inf as it should
    return hi


def f32_from_float(x):
    """Round a Python float (binary64) to the nearest binary32, as a Python float."""
    return float(np.float32(x))


def f32_pattern(x):
    """Python float already representable in binary32 -> its uint32 pattern."""
    return struct.unpack("<I", struct.pack("<f", x))[0]
