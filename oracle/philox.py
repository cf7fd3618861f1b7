"""Philox4x32-10, the counter-based word generator (oracle side).

What the pages fix: the FlyDSL page "Add stochastic rounding and philox RNG
helpers" (Primitives section) describes ``philox_4x32(counter, key)`` as a
counter-based generator that returns four 32-bit words, so a kernel derives
its randomness from an index and a seed and carries no generator state; its
discussion section identifies it with the Philox4_32_10 generator of the
usual libraries, and the "adamw-sr" page (Method and References sections)
keys its rounding randomness with counter-based Philox.

What the pages leave open: the constants and the round function. They are
taken from the published definition (Salmon et al., SC 2011, section 5.2):

  * state: counter (c0, c1, c2, c3) and key (k0, k1), all 32-bit words;
  * one round: the two products  MUL_A * c0  and  MUL_B * c2  are formed in
    full 64-bit width; with (hi_a, lo_a) and (hi_b, lo_b) their halves the
    new counter is  (hi_b ^ c1 ^ k0,  lo_b,  hi_a ^ c3 ^ k1,  lo_a);
  * between two rounds the key is bumped by the Weyl constants
    (k0 += WEYL_A, k1 += WEYL_B, modulo 2**32);
  * 10 rounds; the output is the counter after the last round, words 0..3.
"""

import numpy as np

MUL_A = 0xD2511F53   # multiplier of counter word 0
MUL_B = 0xCD9E8D57   # multiplier of counter word 2
WEYL_A = 0x9E3779B9  # bump of key word 0 (golden ratio)
WEYL_B = 0xBB67AE85  # bump of key word 1 (sqrt(3) - 1)
ROUNDS = 10
_M32 = 0xFFFFFFFF


def philox4x32_10_scalar(ctr, key, rounds=ROUNDS):
    """Pure-Python Philox4x32 on one counter (the generator the FlyDSL pull
    request's Primitives section names; constants and rounds from Salmon et
    al., SC 2011).

    ``ctr``: 4 ints (each taken modulo 2**32); ``key``: 2 ints.
    Returns a tuple of 4 ints in [0, 2**32).
    """
    c0, c1, c2, c3 = (int(x) & _M32 for x in ctr)
    k0, k1 = (int(x) & _M32 for x in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + WEYL_A) & _M32
            k1 = (k1 + WEYL_B) & _M32
        prod_a = MUL_A * c0
        prod_b = MUL_B * c2
        hi_a, lo_a = prod_a >> 32, prod_a & _M32
        hi_b, lo_b = prod_b >> 32, prod_b & _M32
        c0, c1, c2, c3 = hi_b ^ c1 ^ k0, lo_b, hi_a ^ c3 ^ k1, lo_a
    return c0, c1, c2, c3


def philox4x32_10(c0, c1, c2, c3, k0, k1, rounds=ROUNDS):
    """Vectorized Philox4x32 (numpy), the same generator as
    :func:`philox4x32_10_scalar`.

    Counter words and key words broadcast against each other; each is
    converted to uint32 (values must lie in [0, 2**32)). The 32x32->64
    products are taken as uint64 products of zero-extended words.
    Returns four uint32 arrays (words 0..3).
    """
    u32, u64 = np.uint32, np.uint64
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & u64(_M32)
                      for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & u64(_M32)
    k1 = np.asarray(k1, dtype=np.uint64) & u64(_M32)
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
    mask = u64(_M32)
    for r in range(rounds):
        if r:
            k0 = (k0 + u64(WEYL_A)) & mask
            k1 = (k1 + u64(WEYL_B)) & mask
        prod_a = u64(MUL_A) * c0
        prod_b = u64(MUL_B) * c2
        hi_a, lo_a = prod_a >> u64(32), prod_a & mask
        hi_b, lo_b = prod_b >> u64(32), prod_b & mask
        c0, c1, c2, c3 = hi_b ^ c1 ^ k0, lo_b, hi_a ^ c3 ^ k1, lo_a
    return tuple(x.astype(u32) for x in (c0, c1, c2, c3))
