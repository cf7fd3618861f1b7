"""Pins of the oracle's f32 -> bf16 conversions (CPU only).

What pins them:
  * the exact-unbiasedness identity of the FlyDSL page's Tests section: the
    count of random values (out of 65,536) that carry into the kept half is
    the dropped low half read as an integer (brute force);
  * outputs land only on the two bf16 neighbours, checked by comparing real
    values (not bit patterns);
  * random value 0 gives round-toward-zero and 0xFFFF round-away-from-zero
    for inexact inputs, both textbook modes checked by value;
  * the exact mean over all random values equals the input, in rational
    arithmetic;
  * a hand-derived table for Inf, NaN payloads, FLT_MAX, subnormals, zeros;
  * round-to-nearest-even against torch's CPU float32 -> bfloat16 cast (a
    library routine) on every non-NaN input tried.
"""

import json
import multiprocessing
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _value(h):
    """Exact rational value of a finite bf16 pattern, decoded by formula."""
    h = int(h)
    sign = -1 if h & 0x8000 else 1
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))


def _value32(u):
    u = int(u)
    sign = -1 if u & 0x80000000 else 1
    e = (u >> 23) & 0xFF
    f = u & 0x7FFFFF
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f, 1 << 23) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(f, 1 << 23)) * (Fraction(2) ** (e - 127))


ALL_R = np.arange(1 << 16, dtype=np.uint32)


def _count_ups(args):
    hi, lo0, width = args
    L = np.arange(lo0, lo0 + width, dtype=np.uint32)
    u = (np.uint32(hi << 16) | L)[:, None]
    out = oracle.sr_bf16(np.broadcast_to(u, (width, 1 << 16)), ALL_R[None, :])
    return lo0, (out != hi).sum(axis=1)


def test_unbiased_identity_exhaustive():
    """High part 0x3F80 (1.0): every L against every r (2**32 pairs), split
    over the host's cores."""
    claim = json.load(open(os.path.join(GOLDEN, "pages_claims.json")))["sr_unbiased"]
    assert claim["random_values"] == 1 << 16
    hi, width = 0x3F80, 256
    jobs = [(hi, lo0, width) for lo0 in range(0, 1 << 16, width)]
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(min(8, os.cpu_count() or 1)) as pool:
        for lo0, ups in pool.imap_unordered(_count_ups, jobs):
            assert np.array_equal(ups, np.arange(lo0, lo0 + width)), lo0


@pytest.mark.parametrize("hi", [0x0000, 0x3FFF, 0x7F7F, 0xBF80, 0x807F, 0x0080])
def test_unbiased_identity_sampled_high_parts(hi):
    """Other binades (subnormal, mantissa all ones, top finite, negative):
    every r against 512 low parts including the extremes."""
    rng = np.random.default_rng(hi)
    L = np.unique(np.concatenate([
        np.array([0, 1, 2, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF], dtype=np.uint32),
        rng.integers(0, 1 << 16, size=504, dtype=np.uint32)]))
    u = (np.uint32(hi << 16) | L)[:, None]
    out = oracle.sr_bf16(np.broadcast_to(u, (L.size, 1 << 16)), ALL_R[None, :])
    ups = (out != hi).sum(axis=1)
    assert np.array_equal(ups, L)
    assert set(np.unique(out).tolist()) <= {hi, hi + 1}


def test_two_neighbours_by_value_and_textbook_modes():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 32, size=4000, dtype=np.uint64).astype(np.uint32)
    finite = (u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)
    u = u[finite]
    down = oracle.sr_bf16(u, np.zeros_like(u))
    up = oracle.sr_bf16(u, np.full_like(u, 0xFFFF))
    mid = oracle.sr_bf16(u, rng.integers(0, 1 << 16, size=u.size, dtype=np.uint32))
    for x_bits, d, a, m in zip(u.tolist(), down.tolist(), up.tolist(), mid.tolist()):
        x = _value32(x_bits)
        if (a & 0x7F80) == 0x7F80:  # rounding away overflowed to Inf
            assert abs(x) > _value(0x7F7F) and a & 0x7FFF == 0x7F80
            continue
        vd, va = _value(d), _value(a)
        # r = 0: the bf16 value nearest to x toward zero.
        assert abs(vd) <= abs(x) and (vd == 0 or (vd > 0) == (x > 0))
        nxt = _value(d + 1)
        assert abs(nxt) > abs(x)
        if vd == x:
            assert va == x and m == d  # representable values never move
        else:
            # r = 0xFFFF: the bf16 value nearest to x away from zero.
            assert abs(va) > abs(x) and va == nxt
            assert m in (d, d + 1)


def test_exact_mean_over_all_random_values():
    rng = np.random.default_rng(9)
    u = rng.integers(0, 1 << 32, size=1000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, np.array([0x00000001, 0x0000FFFF, 0x3FFFFFFF, 0x7F7F0001,
                                     0x807FFFFF, 0x3F808000], dtype=np.uint32)])
    u = u[((u & np.uint32(0x7F800000)) != np.uint32(0x7F800000))]
    u = u[(u & np.uint32(0x7FFFFFFF)) < np.uint32(0x7F7F0000)]  # no overflow to Inf
    for x_bits in u.tolist():
        out = oracle.sr_bf16(np.full(1 << 16, x_bits, dtype=np.uint32), ALL_R)
        vals, counts = np.unique(out, return_counts=True)
        mean = sum(_value(h) * int(c) for h, c in zip(vals.tolist(), counts.tolist())) / (1 << 16)
        assert mean == _value32(x_bits), hex(x_bits)


# Inputs -> outputs for r16 in (0, 1, 0x7FFF, 0x8000, 0xFFFF), derived by
# hand from the rounding reading (NaN keeps its high half with the quiet bit
# set; everything else adds and truncates).
_TABLE = {
    0x7F800000: [0x7F80] * 5,              # +Inf
    0xFF800000: [0xFF80] * 5,              # -Inf
    0x7FC00000: [0x7FC0] * 5,              # default quiet NaN
    0xFFC00000: [0xFFC0] * 5,
    0x7F800001: [0x7FC0] * 5,              # signalling NaN, payload in low bits
    0x7FFFFFFF: [0x7FFF] * 5,              # all-ones payload: no carry into sign
    0xFFFFFFFF: [0xFFFF] * 5,              # no 32-bit wrap to +0
    0xFF800001: [0xFFC0] * 5,
    0x7F7FFFFF: [0x7F7F, 0x7F80, 0x7F80, 0x7F80, 0x7F80],   # +FLT_MAX
    0xFF7FFFFF: [0xFF7F, 0xFF80, 0xFF80, 0xFF80, 0xFF80],   # -FLT_MAX
    0x7F7F0000: [0x7F7F] * 5,              # bf16 max, exact
    0x00000001: [0x0000, 0x0000, 0x0000, 0x0000, 0x0001],   # smallest subnormal
    0x00008000: [0x0000, 0x0000, 0x0000, 0x0001, 0x0001],   # half a subnormal bf16 step
    0x00000000: [0x0000] * 5,
    0x80000000: [0x8000] * 5,
    0x3F808000: [0x3F80, 0x3F80, 0x3F80, 0x3F81, 0x3F81],   # exactly half way
}
_R = [0, 1, 0x7FFF, 0x8000, 0xFFFF]


def test_special_values_table():
    for x, want in _TABLE.items():
        for r, w in zip(_R, want):
            assert oracle.sr_bf16_scalar(x, r) == w, (hex(x), r)
            assert int(oracle.sr_bf16(np.array([x], np.uint32), np.array([r]))[0]) == w


def test_scalar_equals_vectorized():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    r = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32)
    vs = oracle.sr_bf16(u, r)
    vr = oracle.rn_bf16(u)
    for i in range(u.size):
        assert vs[i] == oracle.sr_bf16_scalar(u[i], r[i])
        assert vr[i] == oracle.rn_bf16_scalar(u[i])


def test_rn_matches_torch_cpu_cast():
    """The oracle's RN against torch's CPU cast (round to nearest even) on
    2**28 random patterns, in slices, plus every low half of nine binades
    (all ties and near-ties)."""
    rng = np.random.default_rng(1)
    lows = np.arange(1 << 16, dtype=np.uint32)
    struct_ = np.concatenate([(np.uint32(h << 16) | lows) for h in
                              (0x0000, 0x0001, 0x3F80, 0x3F81, 0x7F7F, 0x7F7E, 0x8000, 0xBF80, 0xFF7F)])
    slices = [struct_] + [None] * 16
    for k, u in enumerate(slices):
        if u is None:
            u = rng.integers(0, 1 << 32, size=1 << 24, dtype=np.uint64).astype(np.uint32)
        nan = ((u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)) & \
            ((u & np.uint32(0x7FFFFF)) != 0)
        want = torch.from_numpy(u.view(np.float32)).to(torch.bfloat16).view(torch.int16) \
            .numpy().view(np.uint16)
        got = oracle.rn_bf16(u)
        assert np.array_equal(got[~nan], want[~nan]), k
        # torch maps every NaN to one pattern; only NaN-ness is comparable there.
        assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all(got[nan] & 0x7F)


def test_cvt_is_sr_of_the_stream():
    x = np.random.default_rng(2).standard_normal(1000).astype(np.float32)
    base = (1 << 32) - 3
    out = oracle.cvt_f32_bf16_sr(x, 7, 0, base)
    for i in range(x.size):
        r = oracle.random16_scalar(base + i, 7, 0)
        assert out[i] == oracle.sr_bf16_scalar(oracle.f32_bits(x[i:i + 1])[0], r)
