"""Pins for the random-number oracle (oracle/rng.py): the stream words
against the pinned Philox fill layout, exact extremes of the unit
conversion, Box-Muller on hand-picked words, distribution tests against the
exact uniform and normal CDFs, and dropout's special cases and unbiasedness."""

import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import rng


def test_words_follow_the_fill_layout():
    # philox_fill writes call j's four words at 4j .. 4j+3 (pinned elsewhere
    # to the reference generator's values); position p is word p & 3 of call p >> 2.
    seed, step = 0xDEADBEEF, 17
    fill = oracle.philox_fill(64, 1000, seed, step)
    got = rng.words(4 * 1000 + np.arange(256, dtype=np.uint64), seed, step)
    assert np.array_equal(got, fill)


def test_unit_from_word_extremes():
    u = rng.unit_from_word(np.array([0, 0xFF, 0x100, 0x80000000, 0xFFFFFFFF], dtype=np.uint32))
    assert u.dtype == np.float32
    assert u.tolist() == [0.0, 0.0, 2.0 ** -24, 0.5, 1.0 - 2.0 ** -24]


def test_uniform_distribution():
    n = 1 << 20
    u = rng.uniform_f32(n, 3, 1).astype(np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    d = stats.kstest(u, "uniform").statistic
    assert d < 1.95 / math.sqrt(n)           # 0.1% level
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / n)


def test_uniform_range_and_shards():
    y = rng.uniform_f32(10000, 5, 2, base_index=7, low=-2.0, high=3.0)
    assert y.min() >= -2.0 and y.max() <= 3.0
    whole = rng.uniform_f32(10007, 5, 2, low=-2.0, high=3.0)
    assert np.array_equal(y, whole[7:])


def test_box_muller_hand_picked_words():
    r_max = math.sqrt(-2 * math.log(2.0 ** -24))   # u1 at its smallest
    # u1 = 1 -> r = 0 -> both zero
    zc, zs, r = rng.box_muller(np.uint32(0xFFFFFFFF), np.uint32(0x12345678))
    assert r == 0.0 and zc == 0.0 and zs == 0.0
    # u1 = 2**-24 (word 0), u2 = 0 -> (r, 0)
    zc, zs, r = rng.box_muller(np.uint32(0), np.uint32(0))
    assert r == pytest.approx(r_max, rel=1e-15) and zc == r and zs == 0.0
    # u2 = 1/4 -> (0, r); u2 = 1/2 -> (-r, 0)
    zc, zs, r = rng.box_muller(np.uint32(0), np.uint32(0x40000000))
    assert abs(zc) < 1e-15 * r and zs == pytest.approx(r, rel=1e-15)
    zc, zs, r = rng.box_muller(np.uint32(0), np.uint32(0x80000000))
    assert zc == pytest.approx(-r, rel=1e-15) and abs(zs) < 1e-15 * r


def test_normal_distribution():
    n = 1 << 20
    z, _ = rng.normal_f64(n, 11, 4)
    d = stats.kstest(z, "norm").statistic
    assert d < 1.95 / math.sqrt(n)
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    # the two members of a pair are uncorrelated
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 5 / math.sqrt(n / 2)


def test_normal_shards_and_affine():
    whole, _ = rng.normal_f64(1001, 2, 3, mean=1.5, std=0.25)
    part, _ = rng.normal_f64(990, 2, 3, base_index=11, mean=1.5, std=0.25)   # odd start
    assert np.array_equal(part, whole[11:])
    z, _ = rng.normal_f64(1001, 2, 3)
    assert np.allclose(whole, 1.5 + 0.25 * z, rtol=0, atol=1e-15)


def test_dropout_special_cases():
    x = np.array([1.0, -3.0, np.inf, np.nan, 0.0, 2.5] * 2000, dtype=np.float32)
    y, keep = rng.dropout_f32(x, 0.0, 1, 1)
    assert keep.all() and np.array_equal(y.view(np.uint32), x.view(np.uint32))
    p = 0.25
    y, keep = rng.dropout_f32(x, p, 1, 1)
    s = np.float32(1 / (1 - p))
    kx = x[keep]
    with np.errstate(invalid="ignore"):
        assert np.array_equal(y[keep], kx * s, equal_nan=True)
    dropped = x[~keep]
    yd = y[~keep]
    assert np.all(np.signbit(yd[dropped == -3.0])) and np.all(yd[dropped == -3.0] == 0)
    assert np.all(np.isnan(yd[np.isinf(dropped) | np.isnan(dropped)]))
    assert rng.dropout_threshold(0.5) == 2 ** 31
    assert rng.dropout_threshold(0.0) == 0
    with pytest.raises(ValueError):
        rng.dropout_threshold(1.0)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_rate_and_unbiased(p):
    n = 1 << 20
    x = np.full(n, 1.0, dtype=np.float32)
    y, keep = rng.dropout_f32(x, p, 21, 3)
    sd = math.sqrt(p * (1 - p) / n)
    assert abs((1 - keep.mean()) - p) < 5 * sd
    # E[y] = x: the kept fraction times the scale
    assert abs(y.astype(np.float64).mean() - 1.0) < 5 * sd / (1 - p) + 1e-6


def test_dropout_bf16_is_rn_of_f32():
    x = oracle.rn_bf16(oracle.f32_bits(np.linspace(-4, 4, 5000, dtype=np.float32)))
    yb, kb = rng.dropout_bf16(x, 0.3, 8, 9, base_index=5)
    yf, kf = rng.dropout_f32(oracle.bf16_to_f32(x), 0.3, 8, 9, base_index=5)
    assert np.array_equal(kb, kf)
    assert np.array_equal(yb, oracle.rn_bf16(oracle.f32_bits(yf)))
