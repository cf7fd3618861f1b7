"""Philox-based random numbers beyond rounding: uniform and normal draws and
dropout (oracle side).

Source: "Add stochastic rounding and philox RNG helpers" (FlyDSL pull
request), discussion section: the counter-based generator belongs in a
random-number namespace of its own because it also serves dropout and
initialisation. The page gives no formulas for these, so every step below
is a reading (listed with the others in the design notes):

  * Stream: the one the rest of the library uses. Position p (base_index + i
    for element i) takes 32-bit word p & 3 of the Philox4x32-10 call with
    counter (lo32(p >> 2), hi32(p >> 2), 0, 0) and key (seed, step).
  * Uniform: U = (W >> 8) * 2**-24, the top 24 bits of the word as a binary32
    fraction in [0, 1) (exact); a draw in [low, high) is low + (high - low) * U
    evaluated in binary32 (multiply, then add; high - low rounded to binary32
    once).
  * Normal: the Box-Muller transform on the pair of positions (2q, 2q + 1),
    which share a Philox call: u1 = ((W(2q) >> 8) + 1) * 2**-24 in (0, 1],
    u2 = (W(2q + 1) >> 8) * 2**-24, r = sqrt(-2 ln u1); position 2q gets
    r cos(2 pi u2) and 2q + 1 gets r sin(2 pi u2). A draw with mean mu and
    standard deviation s is mu + s * z. The oracle evaluates z in binary64;
    the device evaluates it in binary32 on its log2/sin/cos units, so the
    two are compared within a bound.
  * Dropout with drop probability p in [0, 1): threshold T = floor(p * 2**32)
    (binary64), an element is dropped when W < T (so P(drop) = T / 2**32);
    the output is x * f where f = binary32(1 / (1 - p)) for kept elements and
    f = 0 for dropped ones -- one binary32 multiply (a dropped Inf or NaN
    gives NaN, a dropped negative value -0, as x * (mask * scale) does).
    bf16 inputs are widened exactly and the product is rounded to nearest.

Test infrastructure only (see the package header).
"""

import math

import numpy as np

from .philox import philox4x32_10
from .bf16 import bf16_to_f32, f32_bits, rn_bf16

_M32 = 0xFFFFFFFF
TWO_M24 = np.float32(2.0 ** -24)


def words(positions, seed, step):
    """The 32-bit stream word of every position (uint32), one Philox call
    per position (FlyDSL pull request, discussion: the counter-based
    generator also serves dropout and initialisation; the keying is the
    "adamw-sr" page's Method: key (seed, step), call p >> 2, word p & 3)."""
    p = np.asarray(positions, dtype=np.uint64)
    j = p >> np.uint64(2)
    w = (p & np.uint64(3)).astype(np.intp)
    out = philox4x32_10(j & np.uint64(_M32), j >> np.uint64(32), 0, 0,
                        int(seed) & _M32, int(step) & _M32)
    stacked = np.stack(out, axis=-1)
    return np.take_along_axis(stacked, w[..., None], axis=-1)[..., 0].astype(np.uint32)


def _positions(n, base_index):
    return np.uint64(int(base_index) & 0xFFFFFFFFFFFFFFFF) + np.arange(n, dtype=np.uint64)


def unit_from_word(w):
    """(W >> 8) * 2**-24 in binary32 (exact): the uniform draw of a word in
    [0, 1) (reading: the top 24 bits, so the value is exact in binary32)."""
    return (np.asarray(w, dtype=np.uint32) >> np.uint32(8)).astype(np.float32) * TWO_M24


def uniform_f32(n, seed, step, base_index=0, low=0.0, high=1.0):
    """Uniform draws in [low, high) for initialisation (FlyDSL pull request,
    discussion): f32(low) + f32(high - low) * U, each step rounded in binary32."""
    u = unit_from_word(words(_positions(n, base_index), seed, step))
    width = np.float32(float(high) - float(low))   # rounded once
    return (np.float32(low) + (width * u).astype(np.float32)).astype(np.float32)


def box_muller(w_even, w_odd):
    """(cos-branch, sin-branch) standard normal values in binary64 from the
    words of an (even, odd) position pair."""
    a = (np.asarray(w_even, dtype=np.uint64) >> np.uint64(8)).astype(np.float64)
    b = (np.asarray(w_odd, dtype=np.uint64) >> np.uint64(8)).astype(np.float64)
    u1 = (a + 1.0) * 2.0 ** -24
    u2 = b * 2.0 ** -24
    r = np.sqrt(-2.0 * np.log(u1))
    return r * np.cos(2.0 * np.pi * u2), r * np.sin(2.0 * np.pi * u2), r


def normal_f64(n, seed, step, base_index=0, mean=0.0, std=1.0):
    """Normal draws in binary64 (mean + std * z with z in binary64), plus
    the radius r of each element's pair (for error bounds)."""
    pos = _positions(n, base_index)
    even = pos & ~np.uint64(1)
    w_e = words(even, seed, step)
    w_o = words(even + np.uint64(1), seed, step)
    zc, zs, r = box_muller(w_e, w_o)
    z = np.where((pos & np.uint64(1)) == 0, zc, zs)
    return float(mean) + float(std) * z, r


def dropout_threshold(p):
    """floor(p * 2**32): an element is dropped when its word is below it
    (dropout, FlyDSL pull request discussion), so P(drop) = threshold / 2**32."""
    if not (0.0 <= p < 1.0):
        raise ValueError("p must be in [0, 1)")
    return min(math.floor(p * 2.0 ** 32), _M32)


def dropout_scale(p):
    """The scale of kept elements, 1 / (1 - p) rounded once to binary32."""
    return np.float32(1.0 / (1.0 - p))


def dropout_keep(n, p, seed, step, base_index=0):
    """Boolean keep mask: the word of position base_index + i is at or above
    the drop threshold."""
    return words(_positions(n, base_index), seed, step) >= np.uint32(dropout_threshold(p))


def dropout_f32(x, p, seed, step, base_index=0):
    """(y, keep) for a float32 array x."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    keep = dropout_keep(x.size, p, seed, step, base_index)
    factor = np.where(keep, dropout_scale(p), np.float32(0.0)).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (x * factor).astype(np.float32)
    return y, keep


def dropout_bf16(x_bits, p, seed, step, base_index=0):
    """(y bf16 patterns, keep) for bf16 patterns x_bits."""
    y, keep = dropout_f32(bf16_to_f32(np.asarray(x_bits, dtype=np.uint16).reshape(-1)), p, seed,
                          step, base_index)
    return rn_bf16(f32_bits(y)).astype(np.uint16), keep
