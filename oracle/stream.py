"""Which 16 random bits each element receives (the stream contract).

The "adamw-sr" page (Method section) takes the rounding randomness from a
key made of (seed, step) and from each element's position in the whole
parameter set; its Correctness section states that a parameter updated in
shards, each carrying the position of its first element (base_index),
receives the same bits as when updated in one piece. The FlyDSL page's device tests feed one
Philox word per element, indexed by the global thread index, with the seed
as key.

Readings taken where the pages are silent (each is listed in the design notes):
  * position p = base_index + i, a 64-bit unsigned integer (a 32-bit index
    wraps beyond 2**32 elements, which an 8B-parameter model exceeds);
  * one Philox call serves four consecutive positions: counter
    (lo32(p >> 2), hi32(p >> 2), 0, 0), word number p & 3;
  * key = (seed, lo32(step)), the literal "keyed by (seed, step)";
  * the low 16 bits of the chosen word are the random value.
"""

import numpy as np

from .philox import philox4x32_10, philox4x32_10_scalar

_M32 = 0xFFFFFFFF


def random16_scalar(position, seed, step):
    """The 16-bit random value of one global position (pure Python):
    "adamw-sr" page, Method (key (seed, step), indexed by global position);
    the four words of one call serve four consecutive positions and each
    position takes the low 16 bits of its word."""
    p = int(position) & 0xFFFFFFFFFFFFFFFF
    j = p >> 2
    words = philox4x32_10_scalar((j & _M32, j >> 32, 0, 0),
                                 (int(seed) & _M32, int(step) & _M32))
    return words[p & 3] & 0xFFFF


def random16(positions, seed, step):
    """The 16-bit random values of an array of global positions (numpy), by
    the rule of :func:`random16_scalar`.

    ``positions``: uint64-convertible array. Returns uint32 values < 65536.
    Each element runs its own Philox call (no sharing between neighbours),
    which keeps the indexing plain at four times the work.
    """
    p = np.asarray(positions, dtype=np.uint64)
    j = p >> np.uint64(2)
    w = (p & np.uint64(3)).astype(np.intp)
    words = philox4x32_10(j & np.uint64(_M32), j >> np.uint64(32), 0, 0,
                          int(seed) & _M32, int(step) & _M32)
    stacked = np.stack(words, axis=-1)
    chosen = np.take_along_axis(stacked, w[..., None], axis=-1)[..., 0]
    return chosen & np.uint32(0xFFFF)


def philox_fill(n_counters, counter_base, seed, step, counter_upper=0):
    """The words of ``n_counters`` consecutive Philox calls, flattened (the raw
    word primitive of the FlyDSL pull request's Primitives section).

    Call k uses counter (lo32(c), hi32(c), lo32(counter_upper),
    hi32(counter_upper)) with c = (counter_base + k) mod 2**64 and key
    (seed, step); its four words are elements 4k .. 4k+3 of the result
    (uint32). With counter_upper = 0 these are exactly the calls the stream
    contract above makes.
    """
    c = (np.uint64(int(counter_base) & 0xFFFFFFFFFFFFFFFF)
         + np.arange(int(n_counters), dtype=np.uint64))
    up = int(counter_upper) & 0xFFFFFFFFFFFFFFFF
    words = philox4x32_10(c & np.uint64(_M32), c >> np.uint64(32),
                          up & _M32, up >> 32, int(seed) & _M32, int(step) & _M32)
    return np.stack(words, axis=-1).reshape(-1)
