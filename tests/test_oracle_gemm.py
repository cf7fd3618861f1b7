"""Pins for the GEMM side of the oracle (oracle/gemm.py), against facts that
do not come from the oracle itself: exact rational arithmetic, hand-computed
products, structural identities (identity and all-ones operands catch a
transposed operand or a wrong index), f32 summation in several orders
against the error bound, and the scalar generator for the output keying."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import gemm as og


def _bf16_bits(x):
    x = np.asarray(x, dtype=np.float32)
    return oracle.rn_bf16(oracle.f32_bits(x)).astype(np.uint16)


def _randn_bits(rng, shape):
    return _bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_hand_computed_2x2():
    # A = [[1, 2], [3, 4]], B = [[5, 6], [7, 8]]: C = A B^T = [[17, 23], [39, 53]]
    a = _bf16_bits([[1, 2], [3, 4]])
    b = _bf16_bits([[5, 6], [7, 8]])
    assert og.gemm_exact(a, b).tolist() == [[17.0, 23.0], [39.0, 53.0]]
    assert og.gemm_exact_scalar(a, b) == [[17, 23], [39, 53]]


def test_identity_and_ones_fix_the_operand_roles():
    rng = np.random.default_rng(3)
    b = _randn_bits(rng, (5, 8))                    # N x K
    eye = _bf16_bits(np.eye(8))                     # A = I (M = K = 8)
    bv = oracle.bf16_to_f32(b).astype(np.float64)
    # C[m][n] = B[n][m]
    assert np.array_equal(og.gemm_exact(eye, b), bv.T)
    ones = _bf16_bits(np.ones((3, 8)))
    # C[m][n] = sum_k B[n][k], the same for every m
    want = np.array([sum(Fraction(float(v)) for v in row) for row in bv], dtype=object)
    got = og.gemm_exact(ones, b)
    for m in range(3):
        assert [Fraction(float(v)) for v in got[m]] == list(want)


def test_matches_exact_rationals():
    rng = np.random.default_rng(11)
    a = _randn_bits(rng, (4, 24))
    b = _randn_bits(rng, (6, 24))
    exact = og.gemm_exact_scalar(a, b)
    got = og.gemm_exact(a, b)
    absp = og.abs_products(a, b)
    for i in range(4):
        for j in range(6):
            err = abs(Fraction(float(got[i, j])) - exact[i][j])
            assert err <= Fraction(24 * 2.0 ** -53) * Fraction(float(absp[i, j])) * 2
            # fsum of the exact products is the correctly rounded sum
            assert og.gemm_dot(a[i], b[j]) == float(exact[i][j])


def test_integer_inputs_are_exact():
    rng = np.random.default_rng(5)
    a = _bf16_bits(rng.integers(-8, 9, size=(7, 40)).astype(np.float32))
    b = _bf16_bits(rng.integers(-8, 9, size=(9, 40)).astype(np.float32))
    exact = og.gemm_exact_scalar(a, b)
    assert og.gemm_exact(a, b).tolist() == [[float(v) for v in row] for row in exact]


def _f32_sum(products, order):
    """Sums the columns of a (K, cells) float32 array of exact products in
    float32, in a given order of the K terms."""
    if order == "seq":
        acc = np.zeros(products.shape[1], np.float32)
        for t in range(products.shape[0]):
            acc = np.float32(acc + products[t])
        return acc
    if order == "rev":
        return _f32_sum(products[::-1], "seq")
    if order == "tree":
        x = products
        while x.shape[0] > 1:
            if x.shape[0] % 2:
                x = np.concatenate([x, np.zeros((1, x.shape[1]), np.float32)])
            x = np.float32(x[0::2] + x[1::2])
        return x[0]
    if order == "blocks16":  # partial sums of 16 terms, then the partials in order
        parts = [_f32_sum(products[s:s + 16], "tree") for s in range(0, products.shape[0], 16)]
        return _f32_sum(np.stack(parts), "seq")
    raise ValueError(order)


@pytest.mark.parametrize("order", ["seq", "rev", "tree", "blocks16"])
def test_f32_bound_holds_for_summation_orders(order):
    rng = np.random.default_rng(19)
    k = 256
    a = _randn_bits(rng, (16, k))
    b = _randn_bits(rng, (12, k))
    av = oracle.bf16_to_f32(a)
    bv = oracle.bf16_to_f32(b)
    # products of bf16 values are exact in float32 (16 significant bits)
    prods = (av[:, None, :] * bv[None, :, :]).reshape(-1, k).T.astype(np.float32)
    assert np.array_equal(prods.astype(np.float64),
                          (av[:, None, :].astype(np.float64) * bv[None, :, :]).reshape(-1, k).T)
    got = _f32_sum(prods, order).reshape(16, 12).astype(np.float64)
    err = np.abs(got - og.gemm_exact(a, b))
    assert np.all(err <= og.f32_sum_bound(a, b))


def test_f32_bound_catches_a_dropped_term():
    rng = np.random.default_rng(23)
    k = 64
    a = _randn_bits(rng, (32, k))
    b = _randn_bits(rng, (32, k))
    exact = og.gemm_exact(a, b)
    a_drop = a.copy()
    a_drop[:, 5] = 0
    wrong = og.gemm_exact(a_drop, b)
    caught = np.abs(wrong - exact) > og.f32_sum_bound(a, b)
    # a single product can be tiny, so not every element shows it; every
    # row and every column of the result does
    assert caught.mean() > 0.95
    assert caught.any(axis=1).all() and caught.any(axis=0).all()


def test_round_keys_output_element_by_row_major_position():
    rng = np.random.default_rng(29)
    m, n, seed, step, base = 3, 5, 77, 4, 7
    c = rng.standard_normal((m, n)).astype(np.float32)
    got = og.gemm_round(c, "sr", seed=seed, step=step, base_index=base)
    bits = oracle.f32_bits(c)
    for i in range(m):
        for j in range(n):
            r = oracle.random16_scalar(base + i * n + j, seed, step)
            assert got[i, j] == oracle.sr_bf16_scalar(int(bits[i, j]), r)
    rn = og.gemm_round(c, "rn")
    for i in range(m):
        for j in range(n):
            assert rn[i, j] == oracle.rn_bf16_scalar(int(bits[i, j]))


def test_round_rows_alone_with_offset_base():
    rng = np.random.default_rng(31)
    c = rng.standard_normal((10, 7)).astype(np.float32)
    whole = og.gemm_round(c, "sr", seed=5, step=2, base_index=12)
    part = og.gemm_round(c[3:8], "sr", seed=5, step=2, base_index=12 + 3 * 7)
    assert np.array_equal(part, whole[3:8])


def test_round_at_matches_whole():
    rng = np.random.default_rng(37)
    c = rng.standard_normal((9, 13)).astype(np.float32)
    whole = og.gemm_round(c, "sr", seed=9, step=1, base_index=3)
    rows = rng.integers(0, 9, 20)
    cols = rng.integers(0, 13, 20)
    got = og.gemm_round_at(c[rows, cols], rows, cols, 13, 9, 1, base_index=3)
    assert np.array_equal(got, whole[rows, cols])
