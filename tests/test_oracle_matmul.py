"""Pins of the matrix-product oracle (C = A B^T) to facts other than itself:
brute-force loops, closed forms (identity, all-ones, rank one) and a planted
mistake."""

import numpy as np
import pytest

from oracle import brute_force_matmul_nt, matmul_nt


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (3, 2, 5), (4, 7, 3), (2, 9, 8)])
def test_matches_brute_force(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    a, b = rng.standard_normal((m, k)), rng.standard_normal((n, k))
    np.testing.assert_allclose(matmul_nt(a, b), np.array(brute_force_matmul_nt(a, b)),
                               rtol=1e-13, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((6, 4))
    # B = I: C = A (the transpose of the identity is itself)
    np.testing.assert_array_equal(matmul_nt(a, np.eye(4)), a)
    # B all ones: each column of C is the row sums of A
    np.testing.assert_allclose(matmul_nt(a, np.ones((3, 4))), np.repeat(a.sum(1, keepdims=True), 3, 1),
                               rtol=1e-14, atol=1e-14)
    # rank one: A = u x^T, B = v x^T gives C = (x . x) u v^T
    u, v, x = rng.standard_normal(6), rng.standard_normal(5), rng.standard_normal(4)
    np.testing.assert_allclose(matmul_nt(np.outer(u, x), np.outer(v, x)), (x @ x) * np.outer(u, v),
                               rtol=1e-13, atol=1e-13)


def test_rejects_mismatched_reduction():
    with pytest.raises(ValueError):
        matmul_nt(np.zeros((2, 3)), np.zeros((2, 4)))


def test_pins_catch_transposed_operand():
    rng = np.random.default_rng(6)
    a, b = rng.standard_normal((3, 3)), rng.standard_normal((3, 3))
    mutant = a @ b  # forgets the transpose
    assert not np.allclose(mutant, np.array(brute_force_matmul_nt(a, b)))
