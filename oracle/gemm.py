"""bf16 GEMM with a bf16 output rounded by SR or RN (oracle side).

Source: "Add stochastic rounding and philox RNG helpers" (FlyDSL pull
request), Consumer section: a bf16 GEMM accumulates in f32 and converts the f32
accumulator to bf16, by round-to-nearest (the default) or by stochastic
rounding keyed per output element from a seed; Tests section: the SR output
stays within tolerance of RN, changes with the seed and is reproducible for
a fixed seed.

Readings where the page leaves a step open:
  * Layout: C = A B^T with A (M x K) and B (N x K), K contiguous in both
    (a linear layer y = x W^T). C[m][n] = sum_k A[m][k] B[n][k].
  * Keying: output element (m, n) takes stream position base_index + m*N + n
    under key (seed, step): the stream and rule of the stand-alone
    conversion, so rounding inside the GEMM equals converting its f32 result.
  * The page fixes no f32 summation order, so the oracle gives two things:
    the exact product (every bf16 x bf16 product is exact in binary64, and
    the sums are formed in binary64: exact for small-integer inputs, within
    K * 2**-53 * sum|a b| otherwise), with a bound any f32 summation order
    meets; and the rounding of a given f32 result, which is exact.

Test infrastructure only (see the package header).
"""

import math
from fractions import Fraction

import numpy as np

from .bf16 import bf16_to_f32, f32_bits, sr_bf16, rn_bf16
from .stream import random16

U32 = 2.0 ** -24   # unit roundoff of binary32


def _values(bits):
    return bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def gemm_exact(a_bits, b_bits):
    """C = A B^T in binary64 from bf16 patterns A (M x K) and B (N x K).

    Products are exact in binary64 (8-bit by 8-bit significands); the sums
    are exact when every partial sum fits 53 bits (true for the small-integer
    inputs the exact tests use)."""
    a = _values(a_bits)
    b = _values(b_bits)
    return a @ b.T


def gemm_exact_scalar(a_bits, b_bits):
    """The same product with exact rational arithmetic, for tiny inputs:
    a list of rows of Fractions."""
    a = _values(a_bits)
    b = _values(b_bits)
    m, k = a.shape
    n = b.shape[0]
    return [[sum((Fraction(float(a[i, t])) * Fraction(float(b[j, t])) for t in range(k)),
                 Fraction(0)) for j in range(n)] for i in range(m)]


def gemm_dot(a_row_bits, b_row_bits):
    """One output element, correctly rounded to binary64 (math.fsum of exact
    products): for sampled checks of outputs too large to form whole."""
    a = _values(a_row_bits)
    b = _values(b_row_bits)
    return math.fsum((a * b).tolist())


def abs_products(a_bits, b_bits):
    """sum_k |A[m][k]| |B[n][k]| (binary64)."""
    return np.abs(_values(a_bits)) @ np.abs(_values(b_bits)).T


def f32_sum_bound(a_bits, b_bits):
    """Bound on |C_f32 - C| for an f32 result formed from the exact
    products by K - 1 additions in any order, each rounded faithfully
    (error below one unit in the last place, so at most 2u relative): the
    first-order bound 2 (K - 1) u sum|a b|, plus a 1% margin for the
    second-order terms and the binary64 error of the reference itself."""
    k = np.asarray(a_bits).shape[1]
    return 1.01 * 2.0 * max(k - 1, 1) * U32 * abs_products(a_bits, b_bits)


def gemm_round(c_f32, rounding, seed=0, step=0, base_index=0):
    """bf16 patterns of an M x N f32 result: "rn" or "sr" (position
    base_index + m*N + n, key (seed, step)). "Add stochastic rounding and
    philox RNG helpers", Consumer section: the f32 accumulator goes to bf16 by SR
    keyed per output element, RN by default; reading: the position is the
    row-major index."""
    c = np.asarray(c_f32, dtype=np.float32)
    bits = f32_bits(c.reshape(-1))
    if rounding == "rn":
        out = rn_bf16(bits)
    elif rounding == "sr":
        pos = (np.uint64(int(base_index) & 0xFFFFFFFFFFFFFFFF)
               + np.arange(bits.size, dtype=np.uint64))
        out = sr_bf16(bits, random16(pos, seed, step))
    else:
        raise ValueError("rounding must be 'rn' or 'sr'")
    return out.reshape(c.shape)


def gemm_round_at(c_f32_values, rows, cols, n_cols, seed, step, base_index=0):
    """SR patterns of selected elements (the rule of :func:`gemm_round`):
    c_f32_values[i] is output element (rows[i], cols[i]) of a result with
    n_cols columns."""
    bits = f32_bits(np.asarray(c_f32_values, dtype=np.float32).reshape(-1))
    pos = (np.uint64(int(base_index) & 0xFFFFFFFFFFFFFFFF)
           + np.asarray(rows, dtype=np.uint64) * np.uint64(n_cols)
           + np.asarray(cols, dtype=np.uint64))
    return sr_bf16(bits, random16(pos, seed, step))
