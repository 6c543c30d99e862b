"""Pins of the float64 CPU oracle to facts other than itself.

Each test checks the oracle against something the pages or the mathematics
fix independently: brute force with Python loops, finite differences, closed
forms for degenerate inputs (one key, two keys, constant keys, scale 0),
library routines (scipy softmax / logsumexp / expit), the online-softmax
update rule of the Lecture 17 page §8.3, and invariances. The last block
plants typical mistakes in copies of the oracle and checks that at least one
pin catches each of them.
"""

import numpy as np
import pytest
from scipy.special import expit, logsumexp, softmax

from oracle import (
    attention_backward,
    attention_forward,
    brute_force_backward,
    brute_force_forward,
    online_softmax_forward,
)


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


# --------------------------------------------------------------------------
# brute force (pure Python loops, math.exp) on tiny shapes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 5])
@pytest.mark.parametrize("d", [1, 2, 4])
def test_forward_matches_brute_force(n, d):
    rng = np.random.default_rng(100 + 10 * n + d)
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    scale = 1.0 / np.sqrt(d)
    o, lse = attention_forward(q, k, v, scale)
    ob, lseb = brute_force_forward(q, k, v, scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(lseb), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("n,d", [(1, 2), (2, 1), (3, 2), (5, 4)])
def test_backward_matches_finite_differences(n, d):
    rng = np.random.default_rng(7 * n + d)
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = attention_backward(q, k, v, do, scale)
    fq, fk, fv = (np.array(g) for g in brute_force_backward(q, k, v, do, scale))
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(got, want, rtol=1e-7, atol=1e-8)


def test_cross_attention_shapes_brute_force():
    # Nq != Nk and d_v != d_k: the definition does not need them equal.
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 3, 4), _rand(rng, 5, 4), _rand(rng, 5, 2)
    o, lse = attention_forward(q, k, v, 0.3)
    ob, lseb = brute_force_forward(q, k, v, 0.3)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(lseb), rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_key():
    rng = np.random.default_rng(11)
    q, k, v, do = (_rand(rng, 1, 8) for _ in range(4))
    scale = 0.37
    o, lse = attention_forward(q, k, v, scale)
    assert np.array_equal(o, v)
    np.testing.assert_allclose(lse, scale * (q @ k.T)[:, 0], rtol=0, atol=1e-15)
    dq, dk, dv = attention_backward(q, k, v, do, scale)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv, do)


def test_two_keys_is_logistic():
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 6, 4), _rand(rng, 2, 4), _rand(rng, 2, 4)
    scale = 0.5
    s = scale * q @ k.T
    sig = expit(s[:, 0] - s[:, 1])  # P_i1 = logistic(S_i1 - S_i2)
    o, lse = attention_forward(q, k, v, scale)
    want = sig[:, None] * v[0] + (1.0 - sig)[:, None] * v[1]
    np.testing.assert_allclose(o, want, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("n", [4, 33, 128])
def test_constant_keys(n):
    rng = np.random.default_rng(n)
    d = 8
    q, v, do = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    kvec = _rand(rng, d)
    k = np.tile(kvec, (n, 1))
    scale = 1.0 / np.sqrt(d)
    o, lse = attention_forward(q, k, v, scale)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, scale * q @ kvec + np.log(n), rtol=1e-14, atol=1e-14)
    dq, dk, dv = attention_backward(q, k, v, do, scale)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv, np.tile(do.sum(axis=0) / n, (n, 1)), rtol=1e-13, atol=1e-14)
    # P = 1/n everywhere, so dS_ij = (dO_i . (v_j - vbar)) / n and
    # dK_j = (scale / n) * sum_i (dO_i . (v_j - vbar)) q_i.
    vbar = v.mean(axis=0)
    want_dk = (scale / n) * ((do @ (v - vbar).T).T @ q)
    np.testing.assert_allclose(dk, want_dk, rtol=1e-12, atol=1e-13)


def test_scale_zero_is_uniform():
    rng = np.random.default_rng(5)
    n, d = 50, 6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v, 0.0)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(n), rtol=0, atol=1e-14)


def test_identity_values_expose_probabilities():
    # V = I (N = d): O = P, which must equal scipy's softmax and sum to 1 per row.
    rng = np.random.default_rng(9)
    n = 16
    q, k = _rand(rng, n, n), _rand(rng, n, n)
    scale = 0.25
    o, lse = attention_forward(q, k, np.eye(n), scale)
    np.testing.assert_allclose(o, softmax(scale * q @ k.T, axis=1), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, logsumexp(scale * q @ k.T, axis=1), rtol=1e-14, atol=1e-14)


def test_lse_matches_logsumexp_with_large_scores():
    # Scores far beyond exp's range: only the max-shifted form survives.
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 64, 32, std=30.0), _rand(rng, 64, 32), _rand(rng, 64, 32)
    o, lse = attention_forward(q, k, v, 1.0)
    s = q @ k.T
    np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=1e-14, atol=1e-12)
    np.testing.assert_allclose(o, softmax(s, axis=1) @ v, rtol=1e-12, atol=1e-13)
    assert np.all(np.isfinite(o))


# --------------------------------------------------------------------------
# the online update of the Lecture 17 page §8.3 against the two-pass definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tile", [1, 7, 64, 200])
def test_online_equals_two_pass(tile):
    rng = np.random.default_rng(tile)
    q = _rand(rng, 2, 3, 200, 16, std=3.0)
    k, v = _rand(rng, 2, 3, 200, 16), _rand(rng, 2, 3, 200, 16)
    scale = 0.25
    o1, l1 = attention_forward(q, k, v, scale)
    o2, l2 = online_softmax_forward(q, k, v, scale, tile)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------

def test_key_shift_invariance():
    rng = np.random.default_rng(31)
    n, d = 40, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    c = _rand(rng, d)
    scale = 0.4
    o1, l1 = attention_forward(q, k, v, scale)
    o2, l2 = attention_forward(q, k + c, v, scale)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + scale * q @ c, rtol=1e-12, atol=1e-12)


def test_key_value_permutation():
    rng = np.random.default_rng(32)
    n, d = 40, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    perm = rng.permutation(n)
    scale = 0.4
    o1, l1 = attention_forward(q, k, v, scale)
    o2, l2 = attention_forward(q, k[perm], v[perm], scale)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-14)
    dq1, dk1, dv1 = attention_backward(q, k, v, do, scale)
    dq2, dk2, dv2 = attention_backward(q, k[perm], v[perm], do, scale)
    np.testing.assert_allclose(dq2, dq1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk2, dk1[perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv2, dv1[perm], rtol=1e-12, atol=1e-13)


def test_backward_sum_rules():
    # Rows of P sum to 1 and rows of dS sum to 0, so sum_j dV_j = sum_i dO_i
    # and sum_j dK_j = 0; also sum_j P_ij dP_ij = dO_i . O_i (the row term).
    rng = np.random.default_rng(33)
    n, d = 64, 16
    q, k, v, do = (_rand(rng, 2, n, d) for _ in range(4))
    scale = 0.25
    o, _ = attention_forward(q, k, v, scale)
    dq, dk, dv = attention_backward(q, k, v, do, scale)
    np.testing.assert_allclose(dv.sum(axis=-2), do.sum(axis=-2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=-2), 0.0, atol=1e-12)
    for b in range(2):
        s = scale * q[b] @ k[b].T
        p = softmax(s, axis=1)
        dp = do[b] @ v[b].T
        np.testing.assert_allclose((p * dp).sum(axis=1), (do[b] * o[b]).sum(axis=1), rtol=1e-12, atol=1e-13)


def test_batched_equals_per_head():
    rng = np.random.default_rng(34)
    q, k, v, do = (_rand(rng, 2, 3, 20, 8) for _ in range(4))
    o, lse = attention_forward(q, k, v, 0.3)
    g = attention_backward(q, k, v, do, 0.3)
    for b in range(2):
        for h in range(3):
            ob, lb = attention_forward(q[b, h], k[b, h], v[b, h], 0.3)
            np.testing.assert_array_equal(o[b, h], ob)
            np.testing.assert_array_equal(lse[b, h], lb)
            gb = attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], 0.3)
            for x, y in zip(g, gb):
                np.testing.assert_array_equal(x[b, h], y)


# --------------------------------------------------------------------------
# planted mistakes: each mutated oracle must fail at least one pin
# --------------------------------------------------------------------------

def _fwd_no_lse_shift(q, k, v, scale):  # forgets +m in LSE
    s = scale * q @ k.T
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ v, np.log(l)[:, 0]


def _fwd_transposed_p(q, k, v, scale):  # uses P^T V
    s = scale * q @ k.T
    p = softmax(s, axis=1)
    return p.T @ v, logsumexp(s, axis=1)


def _fwd_unscaled(q, k, v, scale):  # drops the scale
    s = q @ k.T
    return softmax(s, axis=1) @ v, logsumexp(s, axis=1)


def _fwd_wrong_alpha(q, k, v, scale, tile=3):  # online rule with e^(m' - m) instead of e^(m - m')
    m = np.full((q.shape[0], 1), -np.inf)
    l = np.zeros((q.shape[0], 1))
    o = np.zeros((q.shape[0], v.shape[1]))
    for j0 in range(0, k.shape[0], tile):
        s = scale * q @ k[j0:j0 + tile].T
        m_new = np.maximum(m, s.max(axis=1, keepdims=True))
        alpha = np.exp(np.nan_to_num(m_new - m, posinf=0.0))
        p = np.exp(s - m_new)
        l = alpha * l + p.sum(axis=1, keepdims=True)
        o = alpha * o + p @ v[j0:j0 + tile]
        m = m_new
    return o / l, (m + np.log(l))[:, 0]


def _bwd_no_scale_dk(q, k, v, do, scale):
    dq, dk, dv = attention_backward(q, k, v, do, scale)
    return dq, dk / scale, dv


def _bwd_sign_flip_ds(q, k, v, do, scale):
    s = scale * q @ k.T
    p = softmax(s, axis=1)
    dp = do @ v.T
    ds = p * ((p * dp).sum(axis=1, keepdims=True) - dp)
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _bwd_missing_row_term(q, k, v, do, scale):
    s = scale * q @ k.T
    p = softmax(s, axis=1)
    dp = do @ v.T
    ds = p * dp
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _forward_pins_pass(fwd):
    rng = np.random.default_rng(77)
    q, k, v = _rand(rng, 5, 4), _rand(rng, 5, 4), _rand(rng, 5, 3)
    scale = 0.7
    o, lse = fwd(q, k, v, scale)
    ob, lseb = brute_force_forward(q, k, v, scale)
    return np.allclose(o, ob, rtol=1e-12, atol=1e-13) and np.allclose(lse, lseb, rtol=1e-12, atol=1e-13)


def _backward_pins_pass(bwd):
    rng = np.random.default_rng(78)
    q, k, v, do = (_rand(rng, 4, 3) for _ in range(4))
    scale = 0.7
    got = bwd(q, k, v, do, scale)
    want = brute_force_backward(q, k, v, do, scale)
    return all(np.allclose(a, np.array(b), rtol=1e-7, atol=1e-8) for a, b in zip(got, want))


@pytest.mark.parametrize("mutant", [_fwd_no_lse_shift, _fwd_transposed_p, _fwd_unscaled, _fwd_wrong_alpha])
def test_pins_catch_forward_mutants(mutant):
    assert _forward_pins_pass(lambda q, k, v, s: attention_forward(q, k, v, s))
    assert not _forward_pins_pass(mutant)


@pytest.mark.parametrize("mutant", [_bwd_no_scale_dk, _bwd_sign_flip_ds, _bwd_missing_row_term])
def test_pins_catch_backward_mutants(mutant):
    assert _backward_pins_pass(attention_backward)
    assert not _backward_pins_pass(mutant)


def test_running_max_reading_stale_reference_gives_the_same_softmax():
    # The kernels' reading of the running max (design notes, readings table):
    # any reference value m that keeps 2^(c s - m) finite yields the same O and
    # LSE, because the shift cancels in o / l. Here, in float64 and base 2 as
    # the kernels work, m moves only when a 32-key block's sum exceeds 2^24,
    # and then to that block's max (scaling o, l and the tile's earlier sum by
    # 2^(m_old - m_new)); rows whose scores jump by ~20 and ~60 mid-sequence
    # take that path. The result must equal the two-pass definition.
    rng = np.random.default_rng(31)
    n, d = 300, 16
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    k[150:] *= 6.0
    k[230:] *= 4.0
    v = rng.standard_normal((n, d))
    scale = 1.0 / np.sqrt(d)
    c = scale / np.log(2.0)
    s2 = c * (q @ k.T)  # scores in base-2 units
    m = s2[:, :32].max(axis=1)  # the first block takes its max, as the kernels' first tile does
    l = np.zeros(n)
    o = np.zeros((n, d))
    moves = 0
    for b0 in range(0, n, 32):
        blk = s2[:, b0:b0 + 32]
        with np.errstate(over="ignore"):
            p = np.exp2(blk - m[:, None])
        bs = p.sum(axis=1)
        if not np.all(bs <= 2.0 ** 24):
            m_new = np.maximum(m, blk.max(axis=1))
            alpha = np.exp2(m - m_new)
            o *= alpha[:, None]
            l *= alpha
            m = m_new
            p = np.exp2(blk - m[:, None])
            bs = p.sum(axis=1)
            moves += 1
        l += bs
        o += p @ v[b0:b0 + 32]
    assert moves >= 2  # the jumps did force the max to move
    ro, rl = attention_forward(q, k, v, scale)
    np.testing.assert_allclose(o / l[:, None], ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose((m + np.log2(l)) * np.log(2.0), rl, rtol=1e-12, atol=1e-12)
