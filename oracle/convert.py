"""Stand-alone f32 -> bf16 conversions of a flat array (oracle side).

The FlyDSL page "Add stochastic rounding and philox RNG helpers" (discussion
section) proposes stochastic rounding as a rounding mode of the narrowing
conversion, keyed by a seed. Reading: the conversion of element i uses the
same stream contract as the optimizer's write-back, position base_index + i
under key (seed, step), so converting an f32 result and rounding it inside
the optimizer give the same bits.
"""

import numpy as np

from .bf16 import f32_bits, sr_bf16, rn_bf16
from .stream import random16


def cvt_f32_bf16_sr(x, seed, step, base_index=0):
    """float32 array -> uint16 bf16 patterns by stochastic rounding ("Add
    stochastic rounding and philox RNG helpers", discussion: SR as a rounding
    mode of the conversion; element i takes the bits of position base_index + i
    under (seed, step), the keying of the "adamw-sr" page's Method section)."""
    bits = f32_bits(np.asarray(x, dtype=np.float32).reshape(-1))
    pos = np.uint64(int(base_index) & 0xFFFFFFFFFFFFFFFF) + np.arange(bits.size, dtype=np.uint64)
    return sr_bf16(bits, random16(pos, seed, step))


def cvt_f32_bf16_rn(x):
    """float32 array -> uint16 bf16 patterns, round to nearest even (the
    conversion's default mode in the same discussion)."""
    return rn_bf16(f32_bits(np.asarray(x, dtype=np.float32).reshape(-1)))
