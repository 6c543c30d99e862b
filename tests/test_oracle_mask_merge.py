"""Pins of the oracle's causal masking, unequal query/key lengths and merge rule.

Causal attention is named by the Lecture 17 page (end of §8.3) as part of a
real kernel but not defined there; the reading taken is that the N_q queries
are the last N_q of the N_k key positions (query i sees key j iff
j <= i + N_k - N_q). The pins check that reading by routes that do not go
through the oracle's masking: brute-force loops over the visible keys only,
unmasked attention on the visible prefix of the keys, closed forms for the
first row, causality (a change to an invisible key changes nothing),
finite-difference gradients, and the online update over several tile
widths. The merge of partial results (the partial results written back to
global memory and continued from, CS336 Lecture 5 transcript, FlashAttention
passage) is pinned against brute force over the union of key sets and
against closed forms. The last block plants typical mistakes in copies of
the oracle and checks that a pin catches each of them.
"""

import math

import numpy as np
import pytest

from oracle import (
    attention_backward,
    attention_forward,
    brute_force_backward,
    brute_force_forward,
    merge_partials,
    online_softmax_forward,
)


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


SHAPES = [(1, 1), (3, 3), (5, 5), (2, 5), (5, 2), (4, 7), (7, 4), (1, 6), (6, 1)]


# --------------------------------------------------------------------------
# causal forward against brute force over the visible keys
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nq,nk", SHAPES)
@pytest.mark.parametrize("d", [1, 3])
def test_causal_forward_matches_brute_force(nq, nk, d):
    rng = np.random.default_rng(1000 + 100 * nq + 10 * nk + d)
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d + 1)
    scale = 0.6
    o, lse = attention_forward(q, k, v, scale, causal=True)
    ob, lseb = brute_force_forward(q, k, v, scale, causal=True)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(lseb), rtol=1e-13, atol=1e-14)
    # rows with no visible key: exactly O = 0, LSE = -inf
    empty = max(0, nq - nk)
    assert np.all(o[:empty] == 0) and np.all(np.isneginf(lse[:empty]))
    assert np.all(np.isfinite(lse[empty:]))


@pytest.mark.parametrize("nq,nk", [(16, 16), (5, 16), (16, 5), (1, 9)])
def test_causal_row_is_attention_over_visible_prefix(nq, nk):
    # Row i of causal attention equals plain (unmasked) attention of q_i over
    # the first i + nk - nq + 1 keys: the mask reading, checked by slicing.
    rng = np.random.default_rng(nq * 31 + nk)
    d = 6
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    scale = 0.45
    o, lse = attention_forward(q, k, v, scale, causal=True)
    for i in range(nq):
        n_vis = i + nk - nq + 1
        if n_vis <= 0:
            assert np.all(o[i] == 0) and lse[i] == -np.inf
            continue
        oi, li = attention_forward(q[i:i + 1], k[:n_vis], v[:n_vis], scale)
        np.testing.assert_allclose(o[i], oi[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[i], li[0], rtol=1e-13, atol=1e-14)


def test_causal_first_and_last_rows_closed_form():
    rng = np.random.default_rng(41)
    n, d = 12, 5
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    scale = 0.3
    o, lse = attention_forward(q, k, v, scale, causal=True)
    # the first query sees only the first key
    np.testing.assert_array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(scale * q[0] @ k[0], rel=0, abs=1e-15)
    # the last query sees every key: same as without the mask
    of, lf = attention_forward(q, k, v, scale)
    np.testing.assert_allclose(o[-1], of[-1], rtol=1e-14, atol=1e-15)
    assert lse[-1] == pytest.approx(lf[-1], rel=1e-14)
    # second row: two keys, weights are the logistic of the score gap
    s0, s1 = scale * q[1] @ k[0], scale * q[1] @ k[1]
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    np.testing.assert_allclose(o[1], (1 - w1) * v[0] + w1 * v[1], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("nq,nk", [(10, 10), (4, 10), (10, 4)])
def test_causality_invisible_keys_change_nothing(nq, nk):
    rng = np.random.default_rng(77 + nq + nk)
    d = 4
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    o, lse = attention_forward(q, k, v, 0.5, causal=True)
    for i in range(nq):
        first_hidden = max(0, i + nk - nq + 1)  # first key row i may not see
        if first_hidden >= nk:
            continue
        k2, v2 = k.copy(), v.copy()
        k2[first_hidden:] = _rand(rng, nk - first_hidden, d, std=50.0)
        v2[first_hidden:] = _rand(rng, nk - first_hidden, d, std=50.0)
        o2, lse2 = attention_forward(q, k2, v2, 0.5, causal=True)
        np.testing.assert_array_equal(o2[:i + 1], o[:i + 1])
        np.testing.assert_array_equal(lse2[:i + 1], lse[:i + 1])


def test_causal_with_equal_lengths_differs_from_unmasked():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 8, 4), _rand(rng, 8, 4), _rand(rng, 8, 4)
    o1, _ = attention_forward(q, k, v, 0.5, causal=True)
    o2, _ = attention_forward(q, k, v, 0.5)
    assert not np.allclose(o1[:-1], o2[:-1])


# --------------------------------------------------------------------------
# causal backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nq,nk", [(3, 3), (2, 4), (4, 2), (1, 3)])
def test_causal_backward_matches_finite_differences(nq, nk):
    rng = np.random.default_rng(500 + 10 * nq + nk)
    d = 2
    q, k = _rand(rng, nq, d), _rand(rng, nk, d)
    v, do = _rand(rng, nk, d), _rand(rng, nq, d)
    scale = 0.8
    got = attention_backward(q, k, v, do, scale, causal=True)
    want = brute_force_backward(q, k, v, do, scale, causal=True)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, np.array(b), rtol=1e-7, atol=1e-8)


def test_causal_backward_closed_forms():
    rng = np.random.default_rng(61)
    n, d = 9, 4
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, causal=True)
    # the first query sees one key: its softmax is constant, so dQ_0 = 0
    np.testing.assert_array_equal(dq[0], 0.0)
    # the last key is seen only by the last query, with weight P_{n-1,n-1}
    s = 0.5 * q[-1] @ k.T
    p_last = np.exp(s - s.max())
    p_last /= p_last.sum()
    np.testing.assert_allclose(dv[-1], p_last[-1] * do[-1], rtol=1e-13, atol=1e-14)
    # rows of P sum to 1 over the visible keys, rows of dS to 0
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)


def test_causal_backward_empty_rows_contribute_nothing():
    rng = np.random.default_rng(62)
    nq, nk, d = 7, 3, 4
    q, k, v, do = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d), _rand(rng, nq, d)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, causal=True)
    assert np.all(dq[:nq - nk] == 0)
    # dropping the empty rows leaves dK and dV unchanged
    dq2, dk2, dv2 = attention_backward(q[nq - nk:], k, v, do[nq - nk:], 0.5, causal=True)
    np.testing.assert_allclose(dk, dk2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dv, dv2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dq[nq - nk:], dq2, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# online update with the mask
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tile", [1, 7, 64, 200])
@pytest.mark.parametrize("nq,nk", [(200, 200), (70, 200), (200, 70)])
def test_online_causal_equals_two_pass(tile, nq, nk):
    rng = np.random.default_rng(tile + nq)
    q = _rand(rng, 2, nq, 16, std=3.0)
    k, v = _rand(rng, 2, nk, 16), _rand(rng, 2, nk, 16)
    o1, l1 = attention_forward(q, k, v, 0.25, causal=True)
    o2, l2 = online_softmax_forward(q, k, v, 0.25, tile, causal=True)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2))


# --------------------------------------------------------------------------
# merge of partial results
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cuts", [[3], [1, 4], [2, 3, 5], [0, 6]])
def test_merge_of_brute_force_parts_equals_brute_force(cuts):
    rng = np.random.default_rng(sum(cuts) + 7)
    nq, nk, d = 4, 6, 3
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    scale = 0.7
    edges = [0] + cuts + [nk]
    parts_o, parts_l = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        if a == b:  # an empty key set: O = 0, LSE = -inf
            parts_o.append(np.zeros((nq, d)))
            parts_l.append(np.full(nq, -np.inf))
            continue
        ob, lb = brute_force_forward(q, k[a:b], v[a:b], scale)
        parts_o.append(np.array(ob))
        parts_l.append(np.array(lb))
    o, lse = merge_partials(np.stack(parts_o), np.stack(parts_l))
    ob, lb = brute_force_forward(q, k, v, scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-13, atol=1e-14)


def test_merge_closed_forms():
    rng = np.random.default_rng(90)
    o1, l1 = _rand(rng, 5, 4), _rand(rng, 5)
    # P identical parts: same O, LSE + ln P
    o, lse = merge_partials(np.stack([o1] * 3), np.stack([l1] * 3))
    np.testing.assert_allclose(o, o1, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(lse, l1 + math.log(3), rtol=1e-15, atol=1e-15)
    # an empty part changes nothing
    o, lse = merge_partials(np.stack([o1, np.zeros_like(o1)]), np.stack([l1, np.full(5, -np.inf)]))
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(lse, l1)
    # every part empty: O = 0, LSE = -inf
    o, lse = merge_partials(np.zeros((2, 5, 4)), np.full((2, 5), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # two parts with LSE gap g: weights logistic(g), and huge LSE do not overflow
    o2, l2 = _rand(rng, 5, 4), l1 + 800.0 + rng.standard_normal(5)
    o, lse = merge_partials(np.stack([o1, o2]), np.stack([l1, l2]))
    w2 = 1.0 / (1.0 + np.exp(l1 - l2))
    np.testing.assert_allclose(o, (1 - w2)[:, None] * o1 + w2[:, None] * o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, l2 + np.log1p(np.exp(l1 - l2)), rtol=1e-15, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_merge_of_key_chunks_equals_whole(causal):
    # Split the keys into chunks of 64 (with a ragged last chunk); causal rows
    # whose visible keys stop inside a chunk, or before it, are the cases a
    # split-key kernel meets.
    rng = np.random.default_rng(91 + causal)
    nq, nk, d, w = 48, 200, 8, 64
    q, k, v = _rand(rng, 2, nq, d), _rand(rng, 2, nk, d), _rand(rng, 2, nk, d)
    o_full, l_full = attention_forward(q, k, v, 0.3, causal=causal)
    po, pl = [], []
    for a in range(0, nk, w):
        b = min(nk, a + w)
        # causal visibility by global position: query i sees key j <= i + nk - nq
        s = 0.3 * np.einsum("hid,hjd->hij", q, k[:, a:b])
        if causal:
            vis = np.arange(a, b)[None, :] <= np.arange(nq)[:, None] + (nk - nq)
            s = np.where(vis, s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        ms = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - ms)
        l = e.sum(axis=-1, keepdims=True)
        po.append(np.einsum("hij,hjd->hid", np.divide(e, l, out=np.zeros_like(e), where=l > 0), v[:, a:b]))
        with np.errstate(divide="ignore"):
            pl.append((ms + np.log(l))[..., 0])
    o, lse = merge_partials(np.stack(po), np.stack(pl))
    np.testing.assert_allclose(o, o_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, l_full, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

def _causal_strict(q, k, v, scale):  # j < i instead of j <= i
    nq, nk = q.shape[0], k.shape[0]
    s = scale * q @ k.T
    vis = np.arange(nk)[None, :] < np.arange(nq)[:, None] + (nk - nq)
    s = np.where(vis, s, -np.inf)
    o, lse = np.zeros((nq, v.shape[1])), np.full(nq, -np.inf)
    for i in range(nq):
        if np.isfinite(s[i]).any():
            m = s[i].max()
            e = np.exp(s[i] - m)
            o[i], lse[i] = e @ v / e.sum(), m + np.log(e.sum())
    return o, lse


def _causal_top_left(q, k, v, scale):  # j <= i whatever the lengths
    nq, nk = q.shape[0], k.shape[0]
    s = scale * q @ k.T
    vis = np.arange(nk)[None, :] <= np.arange(nq)[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e @ v / e.sum(axis=1, keepdims=True), (m + np.log(e.sum(axis=1, keepdims=True)))[:, 0]


def _causal_pins_pass(fwd):
    ok = True
    for nq, nk, seed in ((5, 5, 1), (3, 6, 2)):
        rng = np.random.default_rng(seed)
        q, k, v = _rand(rng, nq, 3), _rand(rng, nk, 3), _rand(rng, nk, 3)
        o, lse = fwd(q, k, v, 0.6)
        ob, lb = brute_force_forward(q, k, v, 0.6, causal=True)
        ok &= np.allclose(o, np.array(ob), rtol=1e-12, atol=1e-13)
        ok &= np.allclose(lse, np.array(lb), rtol=1e-12, atol=1e-13)
    return bool(ok)


def _merge_no_renormalise(o_parts, lse_parts):  # weights e^LSE_r without dividing by the total
    w = np.exp(lse_parts)
    return (w[..., None] * o_parts).sum(axis=0), np.log(w.sum(axis=0))


def _merge_average(o_parts, lse_parts):  # plain average of the parts
    return o_parts.mean(axis=0), np.log(np.exp(lse_parts).sum(axis=0))


def _merge_pins_pass(merge):
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 4, 3), _rand(rng, 7, 3), _rand(rng, 7, 3)
    o1, l1 = brute_force_forward(q, k[:2], v[:2], 0.5)
    o2, l2 = brute_force_forward(q, k[2:], v[2:], 0.5)
    o, lse = merge(np.stack([np.array(o1), np.array(o2)]), np.stack([np.array(l1), np.array(l2)]))
    ob, lb = brute_force_forward(q, k, v, 0.5)
    return np.allclose(o, np.array(ob), rtol=1e-12, atol=1e-13) and np.allclose(lse, np.array(lb), rtol=1e-12)


@pytest.mark.parametrize("mutant", [_causal_strict, _causal_top_left])
def test_pins_catch_mask_mutants(mutant):
    assert _causal_pins_pass(lambda q, k, v, s: attention_forward(q, k, v, s, causal=True))
    assert not _causal_pins_pass(mutant)


@pytest.mark.parametrize("mutant", [_merge_no_renormalise, _merge_average])
def test_pins_catch_merge_mutants(mutant):
    assert _merge_pins_pass(merge_partials)
    assert not _merge_pins_pass(mutant)
